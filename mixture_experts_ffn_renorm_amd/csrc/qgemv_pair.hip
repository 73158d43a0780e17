// Per-pair GEMVs on group-quantized expert weights (small batches).
//
// Weight format: the affine group format in the MLX part of the page
// "SGLang issue #22283" (GitHub thread; its kernels are named affine_qmv
// ... gs_64_b_4; 4 and 8 bits are discussed): each row of
// W13 [E, 2I, H] and W2 [E, H, I] holds K codes q in [0, 2^BITS), packed
// least significant first into 32-bit words; every 64 consecutive elements
// of a row share one bf16 scale s and bias b, and w = s * q + b.  The
// thread's open question is a kernel that tolerates a K that is not a
// multiple of its block (K = 1408 = 64 * 22): here a lane takes 16-byte units of codes
// (128 / BITS elements, inside one group) l, l + 64, ... of a row, and a
// ragged last pass simply has fewer units, so any K that is a multiple of
// 64 works.
//
// Per unit a lane forms dq = sum q_i x_i and sx = sum x_i (fp32), and adds
// s * dq + b * sx: the group's scale and bias are applied once per unit
// instead of once per element, and sx is shared by all rows that read the
// same token (or act) row.  The work layout is that of the bf16 per-pair
// GEMVs (sub-section "Small batches skip the sort" of the page "Mixture of
// Experts in vLLM ..."): GEMV 1 pair-major, one act column (a gate row and
// its up row) per wave; GEMV 2 token-major, one slot per wave, 4 output
// columns per workgroup, the waves' sums added in wave order.
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kGroup = 64;
constexpr int kQ1Waves = 4;
constexpr int kQ2Cols = 4;
constexpr int kQMaxWaves = 8;

// bf16 element c of a row of u32x4 chunks
__device__ __forceinline__ float bf16_at(const u32x4* v, int c) {
  const uint32_t w = v[c >> 3][(c & 7) >> 1];
  return (c & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
}

// sum q_i x_i over one 16-byte unit of codes and the matching x elements
template <int BITS>
__device__ __forceinline__ float dot_unit(const u32x4 codes, const u32x4* xv) {
  constexpr int kPer = 32 / BITS;
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  float d = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const float q = (float)((codes[w] >> (BITS * i)) & kMask);
      d = __builtin_fmaf(q, bf16_at(xv, w * kPer + i), d);
    }
  return d;
}

template <int BITS>
__device__ __forceinline__ float sum_unit(const u32x4* xv) {
  constexpr int kEU = 128 / BITS;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kEU; ++c) s += bf16_at(xv, c);
  return s;
}

// 4-bit units on the bf16 dot-2 instruction: a code q in [0, 16) becomes the
// bf16 value 128 + q exactly (exponent of 128, q in the low mantissa bits),
// so a unit's codes turn into bf16 pairs with one shift and one and-or per
// pair, and sum (128 + q_i) x_i - 128 * sum x_i = sum q_i x_i.  Code word w
// holds elements 8w .. 8w + 7; its pair i (i < 4) takes elements i and
// i + 4 (bits 4i and 16 + 4i), and x is regrouped once per unit to match.

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

struct XPairs4 {
  uint32_t y[16];   // (x_i, x_{i+4}) of each 8-element word, as bf16 pairs
  float sx;         // sum of the unit's 32 x
};

__device__ __forceinline__ XPairs4 regroup_x4(const u32x4* xv) {
  XPairs4 r;
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const u32x4 X = xv[w];   // (x0,x1) (x2,x3) (x4,x5) (x6,x7) of word w
    r.y[4 * w + 0] = __builtin_amdgcn_perm(X[2], X[0], 0x05040100u);   // (x0, x4)
    r.y[4 * w + 1] = __builtin_amdgcn_perm(X[2], X[0], 0x07060302u);   // (x1, x5)
    r.y[4 * w + 2] = __builtin_amdgcn_perm(X[3], X[1], 0x05040100u);   // (x2, x6)
    r.y[4 * w + 3] = __builtin_amdgcn_perm(X[3], X[1], 0x07060302u);   // (x3, x7)
#pragma unroll
    for (int j = 0; j < 4; ++j) s = dot2_bf16(X[j], 0x3f803f80u, s);   // (1, 1)
  }
  r.sx = s;
  return r;
}

// sum q_i x_i over one 4-bit unit
__device__ __forceinline__ float dot_unit4(const u32x4 codes, const XPairs4& xp) {
  float d = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      d = dot2_bf16(((codes[w] >> (4 * i)) & 0x000f000fu) | 0x43004300u, xp.y[4 * w + i], d);
  return d - 128.f * xp.sx;
}

__device__ __forceinline__ float bf16_load(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}

// 16 bytes at unit u of a row of units; past the row the load is clamped to
// unit 0 (in bounds; the caller drops that unit's contribution), so that all
// loads of a pass leave back to back with no branch between them
template <bool kStream>
__device__ __forceinline__ u32x4 load_unit(const u32x4* row, int u, int nunit) {
  const u32x4* p = row + (u < nunit ? u : 0);
  return kStream ? __builtin_nontemporal_load(p) : *p;
}

// NC units per lane per pass.
template <int BITS, int NC>
__global__ __launch_bounds__(64 * kQ1Waves) void qgemv_w13_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq,
    const uint16_t* __restrict__ sc, const uint16_t* __restrict__ bi,
    const int32_t* __restrict__ topk_ids, int top_k, int H, int I, uint16_t* __restrict__ act) {
  constexpr int kEU = 128 / BITS;      // elements per unit
  constexpr int kXU = kEU / 8;         // x chunks (16 bytes) per unit
  const int p = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int f = blockIdx.x * kQ1Waves + (threadIdx.x >> 6);
  if (f >= I) return;   // whole wave; no barrier follows
  const int e = topk_ids[p];
  const int t = p / top_k;
  const int nunit = H / kEU, ng = H / kGroup;
  const size_t rg = (size_t)e * 2 * I + f, ru = rg + I;   // gate and up rows
  const u32x4* qg = reinterpret_cast<const u32x4*>(wq) + rg * nunit;
  const u32x4* qu = reinterpret_cast<const u32x4*>(wq) + ru * nunit;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (size_t)t * H);
  float ag = 0.f, au = 0.f;
  for (int base = lane; base < nunit + lane; base += 64 * NC) {
    u32x4 cg[NC], cu[NC], xv[NC][kXU];
    float gs[NC], gb[NC], us[NC], ub[NC];
    // codes, x and the groups' scales and biases all leave before the first
    // wait (the scale loads would otherwise be a second round trip)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int u = base + 64 * c;
      const int g = (u < nunit ? u : 0) * kEU / kGroup;
      cg[c] = load_unit<true>(qg, u, nunit);
      cu[c] = load_unit<true>(qu, u, nunit);
#pragma unroll
      for (int i = 0; i < kXU; ++i)
        xv[c][i] = load_unit<false>(xr, u * kXU + i, nunit * kXU);
      gs[c] = bf16_load(sc + rg * ng + g);
      gb[c] = bf16_load(bi + rg * ng + g);
      us[c] = bf16_load(sc + ru * ng + g);
      ub[c] = bf16_load(bi + ru * ng + g);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bool ok = base + 64 * c < nunit;
      float dg, du;
      if constexpr (BITS == 4) {
        const XPairs4 xp = regroup_x4(xv[c]);
        dg = gs[c] * dot_unit4(cg[c], xp) + gb[c] * xp.sx;
        du = us[c] * dot_unit4(cu[c], xp) + ub[c] * xp.sx;
      } else {
        const float sx = sum_unit<BITS>(xv[c]);
        dg = gs[c] * dot_unit<BITS>(cg[c], xv[c]) + gb[c] * sx;
        du = us[c] * dot_unit<BITS>(cu[c], xv[c]) + ub[c] * sx;
      }
      ag += ok ? dg : 0.f;
      au += ok ? du : 0.f;
    }
  }
  ag = wave_sum(ag);
  au = wave_sum(au);
  if (lane == 0) act[(size_t)p * I + f] = (uint16_t)f32_to_bf16(silu_mul(ag, au));
}

// SPLIT = 2 (rows of at most 32 units): the two half-waves take two of the
// four columns each, so that short rows keep most lanes busy.
template <int BITS, int NC, int SPLIT>
__global__ __launch_bounds__(64 * kQMaxWaves) void qgemv_w2_sum_kernel(
    const uint16_t* __restrict__ act, const uint32_t* __restrict__ wq,
    const uint16_t* __restrict__ sc, const uint16_t* __restrict__ bi,
    const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_weights, int top_k,
    int H, int I, uint16_t* __restrict__ out) {
  constexpr int kEU = 128 / BITS;
  constexpr int kXU = kEU / 8;
  constexpr int kLanes = 64 / SPLIT;        // lanes per column group
  constexpr int kRows = kQ2Cols / SPLIT;    // columns per lane
  __shared__ float red[kQMaxWaves][kQ2Cols];
  const int t = blockIdx.y;
  const int h0 = blockIdx.x * kQ2Cols;   // H % 64 == 0: all columns exist
  const int lane = threadIdx.x & 63;
  const int half = lane / kLanes, ll = lane % kLanes;
  // wave-uniform: the slot's expert id and weight come in through scalar loads
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;    // <= top_k
  const int nunit = I / kEU, ng = I / kGroup;
  float acc[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) acc[r] = 0.f;
  for (int j = w; j < top_k; j += nwaves) {
    const int p = t * top_k + j;
    const int e = topk_ids[p];
    const size_t row0 = (size_t)e * H + h0 + half * kRows;
    const float wt = topk_weights[p];
    const u32x4* ar = reinterpret_cast<const u32x4*>(act + (size_t)p * I);
    float s[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) s[r] = 0.f;
    for (int base = ll; base < nunit + ll; base += kLanes * NC) {
      u32x4 cw[kRows][NC], av[NC][kXU];
      float ws[kRows][NC], wb[kRows][NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int u = base + kLanes * c;
        const int g = (u < nunit ? u : 0) * kEU / kGroup;
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          cw[r][c] = load_unit<true>(reinterpret_cast<const u32x4*>(wq) + (row0 + r) * nunit, u,
                                     nunit);
          ws[r][c] = bf16_load(sc + (row0 + r) * ng + g);
          wb[r][c] = bf16_load(bi + (row0 + r) * ng + g);
        }
#pragma unroll
        for (int i = 0; i < kXU; ++i) av[c][i] = load_unit<false>(ar, u * kXU + i, nunit * kXU);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bool ok = base + kLanes * c < nunit;
        if constexpr (BITS == 4) {
          const XPairs4 xp = regroup_x4(av[c]);
#pragma unroll
          for (int r = 0; r < kRows; ++r) {
            const float d = ws[r][c] * dot_unit4(cw[r][c], xp) + wb[r][c] * xp.sx;
            s[r] += ok ? d : 0.f;
          }
        } else {
          const float sx = sum_unit<BITS>(av[c]);
#pragma unroll
          for (int r = 0; r < kRows; ++r) {
            const float d = ws[r][c] * dot_unit<BITS>(cw[r][c], av[c]) + wb[r][c] * sx;
            s[r] += ok ? d : 0.f;
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[r] = __builtin_fmaf(wt, s[r], acc[r]);
  }
  // sum over the lanes of each column group (DPP, total in its last lane)
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const float v = group_sum_last<kLanes>(acc[r]);
    if (ll == kLanes - 1) red[w][half * kRows + r] = v;
  }
  __syncthreads();
  if (threadIdx.x < kQ2Cols) {
    float v = red[0][threadIdx.x];
    for (int i = 1; i < nwaves; ++i) v += red[i][threadIdx.x];
    out[(size_t)t * H + h0 + threadIdx.x] = (uint16_t)f32_to_bf16(v);
  }
}

// Units per lane per pass for a row of `units` units: one pass up to 256,
// then passes of 256.
int units_per_lane(int units) {
  const int n = (units + 63) / 64;
  return n < 1 ? 1 : (n > 4 ? 4 : n);
}

template <int BITS, int NC>
void launch_q1(const moe_host::QPairGemvArgs& a, hipStream_t s) {
  dim3 grid(moe_host::ceil_div_host(a.I, kQ1Waves), a.M * a.top_k);
  hipLaunchKernelGGL((qgemv_w13_kernel<BITS, NC>), grid, dim3(64 * kQ1Waves), 0, s, a.x, a.w13q,
                     a.w13_scales, a.w13_biases, a.topk_ids, a.top_k, a.H, a.I, a.act);
}

template <int BITS, int NC, int SPLIT = 1>
void launch_q2(const moe_host::QPairGemvArgs& a, hipStream_t s) {
  const int waves = a.top_k < kQMaxWaves ? a.top_k : kQMaxWaves;
  hipLaunchKernelGGL((qgemv_w2_sum_kernel<BITS, NC, SPLIT>), dim3(a.H / kQ2Cols, a.M),
                     dim3(64 * waves), 0, s, a.act, a.w2q, a.w2_scales, a.w2_biases, a.topk_ids,
                     a.topk_weights, a.top_k, a.H, a.I, a.out);
}

template <int BITS>
void launch_q1_nc(const moe_host::QPairGemvArgs& a, hipStream_t s) {
  switch (units_per_lane(a.H * BITS / 128)) {
    case 1: launch_q1<BITS, 1>(a, s); break;
    case 2: launch_q1<BITS, 2>(a, s); break;
    case 3: launch_q1<BITS, 3>(a, s); break;
    default: launch_q1<BITS, 4>(a, s); break;
  }
}

template <int BITS>
void launch_q2_nc(const moe_host::QPairGemvArgs& a, hipStream_t s) {
  // 4-bit units carry 32 act elements each: at most 2 per lane per pass
  // (4 rows x 4 units would spill registers)
  constexpr int kMaxNC = BITS == 4 ? 2 : 4;
  const int n = units_per_lane(a.I * BITS / 128);
  if (a.I * BITS / 128 <= 32) {
    launch_q2<BITS, 1, 2>(a, s);
  } else if (n == 1) {
    launch_q2<BITS, 1>(a, s);
  } else if (n == 2 || kMaxNC == 2) {
    launch_q2<BITS, 2>(a, s);
  } else if constexpr (kMaxNC == 4) {
    if (n == 3) launch_q2<BITS, 3>(a, s); else launch_q2<BITS, 4>(a, s);
  }
}

}  // namespace

namespace moe_host {

hipError_t launch_qpair_gemv1(const QPairGemvArgs& a, hipStream_t s) {
  if (a.bits == 4) launch_q1_nc<4>(a, s); else launch_q1_nc<8>(a, s);
  return hipGetLastError();
}

hipError_t launch_qpair_gemv2(const QPairGemvArgs& a, hipStream_t s) {
  if (a.bits == 4) launch_q2_nc<4>(a, s); else launch_q2_nc<8>(a, s);
  return hipGetLastError();
}

}  // namespace moe_host
