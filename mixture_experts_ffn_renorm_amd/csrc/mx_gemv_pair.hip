// Per-pair GEMVs on MXFP8 experts for very small batches (M*top_k*4 <= E).
//
// Page "Mixture of Experts in vLLM - From First Principles to fused_moe",
// sub-section "Small batches skip the sort": each pair (token t, slot j) is a
// one-row product against its own expert's weights, read from topk_ids[p]
// (no index lists); sub-section "The two index lists": the FP8 GEMM 1 input
// qhidden is a quantized copy of x.  The format is MXFP8 as the OCP
// microscaling specification defines it (named in the MLX part of the page
// "SGLang issue #22283"): per 32 consecutive values along K one E8M0 scale
// and 32 E4M3 elements.
//
// A lane takes 16-byte chunks of codes (16 elements, half a 32-element
// block) l, l + 64, ... of a row; chunks 2b and 2b + 1 of block b sit on
// lanes l and l ^ 1.  Codes are widened to fp32 two at a time with the
// gfx950 FP8 conversion (OCP E4M3), the 16 products of a chunk are added in
// fp32 (each product of two E4M3 values is exact), and the chunk's partial
// sum is scaled by the product of the two block scales (a power of two).
// All loads of a pass come from in-bounds addresses and leave before the
// first wait; chunks past a row's end contribute zero through a select.
//
// GEMV 1: a workgroup owns one pair and 4 act columns, wave w the column
//   f = 4 blockIdx.x + w: gate row f and up row I + f of W13[e] against the
//   MXFP8 codes of x_t (quantized by the top-k launch);
//   act[p, f] = bf16(SiLU(gate) * up).
// GEMV 2: a workgroup owns token t and R output columns, wave w its slots
//   j = w, w + nwaves, ...; the wave quantizes act row p = t*top_k + j to
//   MXFP8 in registers (block amax across the lane pair, the same rounding
//   as the layer's quantizer: nearest E4M3, ties to even, saturated),
//   multiplies it with W2[e] rows h0 .. h0 + R - 1 and adds topk_weights[p]
//   times the result; the waves' sums are added in wave order and rounded
//   once to bf16.
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kG1Waves = 4;
constexpr int kMaxWaves = 8;   // GEMV 2 waves: min(top_k, 8)
constexpr int kG2Rows = 4;     // GEMV 2 output columns per workgroup


// fp32 values of the E4M3 bytes 0, 1 (kHi = false) or 2, 3 (kHi = true) of w
template <bool kHi>
__device__ __forceinline__ f32x2 e4m3x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, kHi);
}

// sum over the 16 E4M3 products of two chunks (fp32)
__device__ __forceinline__ float dot16_e4m3(u32x4 a, u32x4 b) {
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t aq = a[q], bq = b[q];
    const f32x2 a0 = e4m3x2<false>(aq), a1 = e4m3x2<true>(aq);
    const f32x2 b0 = e4m3x2<false>(bq), b1 = e4m3x2<true>(bq);
    s = __builtin_fmaf(a0[0], b0[0], s);
    s = __builtin_fmaf(a0[1], b0[1], s);
    s = __builtin_fmaf(a1[0], b1[0], s);
    s = __builtin_fmaf(a1[1], b1[1], s);
  }
  return s;
}

// 16-byte chunk `ch` of a code row, or (for chunks past the row) its first
// chunk; the caller drops those with a select
__device__ __forceinline__ u32x4 chunk16(const uint8_t* row, int ch, bool ok, bool stream) {
  const u32x4* p = reinterpret_cast<const u32x4*>(row + (size_t)(ok ? ch : 0) * 16);
  return stream ? __builtin_nontemporal_load(p) : *p;
}

template <int NC>
__global__ __launch_bounds__(64 * kG1Waves) void mx_gemv_w13_kernel(
    const uint8_t* __restrict__ qx, const uint8_t* __restrict__ qxs,
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ w13s,
    const int32_t* __restrict__ ids, int top_k, int H, int I, uint16_t* __restrict__ act) {
  const int p = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int f = blockIdx.x * kG1Waves + (threadIdx.x >> 6);
  if (f >= I) return;   // whole wave; no barrier follows
  const int e = ids[p];
  const int nchunk = H / 16, nb = H / 32;
  const uint8_t* xrow = qx + (size_t)(p / top_k) * H;
  const uint8_t* xsc = qxs + (size_t)(p / top_k) * nb;
  const uint8_t* grow = w13 + ((size_t)e * 2 * I + f) * H;
  const uint8_t* urow = grow + (size_t)I * H;
  const uint8_t* gsc = w13s + ((size_t)e * 2 * I + f) * nb;
  const uint8_t* usc = gsc + (size_t)I * nb;
  float accg = 0.f, accu = 0.f;
  for (int base = lane; base < nchunk + lane; base += 64 * NC) {
    u32x4 xv[NC], gv[NC], uv[NC];
    int sx[NC], sg[NC], su[NC];
    bool ok[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = base + 64 * c;
      ok[c] = ch < nchunk;
      const int bl = ok[c] ? ch >> 1 : 0;
      xv[c] = chunk16(xrow, ch, ok[c], false);
      gv[c] = chunk16(grow, ch, ok[c], true);
      uv[c] = chunk16(urow, ch, ok[c], true);
      sx[c] = xsc[bl];
      sg[c] = gsc[bl];
      su[c] = usc[bl];
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float dg = dot16_e4m3(gv[c], xv[c]);
      const float du = dot16_e4m3(uv[c], xv[c]);
      accg += ok[c] ? __builtin_ldexpf(dg, sg[c] + sx[c] - 254) : 0.f;
      accu += ok[c] ? __builtin_ldexpf(du, su[c] + sx[c] - 254) : 0.f;
    }
  }
  accg = wave_sum(accg);
  accu = wave_sum(accu);
  if (lane == 0) act[(size_t)p * I + f] = (uint16_t)f32_to_bf16(silu_mul(accg, accu));
}

template <int NC>
__global__ __launch_bounds__(64 * kMaxWaves) void mx_gemv_w2_sum_kernel(
    const uint16_t* __restrict__ act, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ w2s, const int32_t* __restrict__ topk_ids,
    const float* __restrict__ topk_weights, int top_k, int H, int I,
    uint16_t* __restrict__ out) {
  constexpr int R = kG2Rows;
  __shared__ float red[kMaxWaves][R];
  const int t = blockIdx.y;
  const int h0 = blockIdx.x * R;   // H % 8 == 0 and R divides 8: all R rows exist
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;   // <= top_k
  const int nchunk = I / 16, nb = I / 32;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  for (int j = w; j < top_k; j += nwaves) {
    const int p = t * top_k + j;
    const float wt = topk_weights[p];
    const uint16_t* arow = act + (size_t)p * I;
    const int e = topk_ids[p];
    const uint8_t* wrow = w2 + ((size_t)e * H + h0) * I;
    const uint8_t* wsc = w2s + ((size_t)e * H + h0) * nb;
    for (int base = lane; base < nchunk + lane; base += 64 * NC) {
      u32x4 av[NC][2], wv[NC][R];
      int sw[NC][R];
      bool ok[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int ch = base + 64 * c;
        ok[c] = ch < nchunk;
        const int cc = ok[c] ? ch : 0;
        const u32x4* ap = reinterpret_cast<const u32x4*>(arow + (size_t)cc * 16);
        av[c][0] = ap[0];
        av[c][1] = ap[1];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          wv[c][r] = chunk16(wrow + (size_t)r * I, ch, ok[c], true);
          sw[c][r] = wsc[(size_t)r * nb + (cc >> 1)];
        }
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        // quantize this lane's 16 act values with the block's shared exponent
        // (the block's other 16 sit on lane ^ 1; I % 32 == 0, so a block's
        // two chunks are both inside the row or both past it)
        float v[16];
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t u = av[c][q >> 2][q & 3];
          v[2 * q] = bf16_lo(u);
          v[2 * q + 1] = bf16_hi(u);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, kWave));
        const int shared = mx_shared_exp(amax);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          v[i] = __builtin_copysignf(
              e4m3_round_mag(__builtin_ldexpf(__builtin_fabsf(v[i]), -shared)), v[i]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float d = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x2 lo = e4m3x2<false>(wv[c][r][q]), hi = e4m3x2<true>(wv[c][r][q]);
            d = __builtin_fmaf(lo[0], v[4 * q], d);
            d = __builtin_fmaf(lo[1], v[4 * q + 1], d);
            d = __builtin_fmaf(hi[0], v[4 * q + 2], d);
            d = __builtin_fmaf(hi[1], v[4 * q + 3], d);
          }
          acc[r] += ok[c] ? wt * __builtin_ldexpf(d, shared + sw[c][r] - 127) : 0.f;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == 0) red[w][r] = v;
  }
  __syncthreads();
  if (threadIdx.x < R) {
    float v = red[0][threadIdx.x];
    for (int i = 1; i < nwaves; ++i) v += red[i][threadIdx.x];
    out[(size_t)t * H + h0 + threadIdx.x] = (uint16_t)f32_to_bf16(v);
  }
}

// chunks of 16 codes per lane per pass: enough to cover K in one pass up to
// 4096, then passes of 4096
int mx_chunks_per_lane(int K) {
  const int n = (K / 16 + 63) / 64;
  return n < 1 ? 1 : (n > 4 ? 4 : n);
}

template <int NC>
void launch_w13(const moe_host::MxPairGemvArgs& a, hipStream_t s) {
  dim3 grid(moe_host::ceil_div_host(a.I, kG1Waves), a.M * a.top_k);
  hipLaunchKernelGGL(mx_gemv_w13_kernel<NC>, grid, dim3(64 * kG1Waves), 0, s, a.qx, a.qx_scales,
                     a.w13, a.w13_scales, a.topk_ids, a.top_k, a.H, a.I, a.act);
}

template <int NC>
void launch_w2(const moe_host::MxPairGemvArgs& a, hipStream_t s) {
  const int waves = a.top_k < kMaxWaves ? a.top_k : kMaxWaves;
  hipLaunchKernelGGL(mx_gemv_w2_sum_kernel<NC>, dim3(a.H / kG2Rows, a.M), dim3(64 * waves), 0, s,
                     a.act, a.w2, a.w2_scales, a.topk_ids, a.topk_weights, a.top_k, a.H, a.I,
                     a.out);
}

}  // namespace

namespace moe_host {

hipError_t launch_mx_pair_gemv1(const MxPairGemvArgs& a, hipStream_t s) {
  switch (mx_chunks_per_lane(a.H)) {
    case 1: launch_w13<1>(a, s); break;
    case 2: launch_w13<2>(a, s); break;
    case 3: launch_w13<3>(a, s); break;
    default: launch_w13<4>(a, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_mx_pair_gemv2(const MxPairGemvArgs& a, hipStream_t s) {
  switch (mx_chunks_per_lane(a.I)) {
    case 1: launch_w2<1>(a, s); break;
    case 2: launch_w2<2>(a, s); break;
    case 3: launch_w2<3>(a, s); break;
    default: launch_w2<4>(a, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe_host
