// Weight-streaming grouped GEMMs on group-quantized expert weights, for
// batches past the per-pair GEMVs (more than one pair per expert on
// average, so each expert's codes should be read once per block of pairs,
// not once per pair).
//
// Weight format: the affine group format of the MLX part of the page
// "SGLang issue #22283" (affine_qmv ... gs_64_b_4): K codes q per row,
// packed least significant first into 32-bit words (4 or 8 bits), and per
// 64 consecutive elements one bf16 scale s and bias b, w = s q + b.  The
// GEMMs are those of the page "Mixture of Experts in vLLM - From First
// Principles to fused_moe": index lists with blocks of 16 pairs
// (sub-section "The two index lists"), GEMM 1 with SiLU(gate) * up written
// to act in pair order ("One GEMM 1 program, step by step"), GEMM 2 into
// weighted fp32 pair-order rows that a small kernel sums per token ("The
// rest of the layer stays in pair order", section "Put the results back,
// and combine them per token").
//
// Dequantizing on the matrix cores: within a group, sum_k w_k x_k =
// s * sum_k q_k x_k + b * sum_k x_k.  Codes widen exactly to bf16 (8 bits:
// q itself; 4 bits: 128 + q, whose bf16 pattern is 0x4300 | q, so each pair
// of codes is one byte permute and one or), the 16x16x32 bf16 MFMA forms
// D = sum (q [+ 128]) x over the group's two k steps, a third MFMA with an
// all-ones A operand forms S = sum x, and each lane then adds
// s D + (b [- 128 s]) S to its fp32 accumulators -- fp32 throughout, no
// weight is rounded.  (The 128 offset costs a relative error near 2^-24
// times 128 / |q - mean|, far below bf16.)
//
// Streaming: persistent workgroups (two per CU), each XCD walking one
// contiguous range of tiles; per tile, K streams through a 3-stage LDS ring
// filled by global_load_lds (16-byte copies of codes and of the gathered x
// or act rows, 4-byte copies of the slice's scales and biases; codes with
// the non-temporal policy).  Every wave issues the same number of copies
// per slice, so one vmcnt count serves all.  Pads (id >= M*top_k) and the
// K tail copy the zeroed page, whose codes, scales and biases are all zero.
// GEMM 1 stores SiLU(gate) * up as bf16 act; GEMM 2 stores topk_weights[p]
// times its tile as fp32 partial rows.  H and I must be multiples of 128
// (the 4-byte scale copies stay aligned); other shapes run the per-pair
// GEMVs.
#include <algorithm>
#include <type_traits>

#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kBM = 16;          // pairs per block
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kStages = 3;
constexpr int kGroup = 64;       // elements per scale / bias

__device__ __forceinline__ void copy_lds4(const void* src, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)lds_dst, 4, 0, 0);
}

// Eight 4-bit codes (one 32-bit word, element i in bits 4i..4i+3) as eight
// bf16 values 128 + q, two per dword in element order: lo holds the even
// elements' nibbles as bytes, h1 / h2 the odd ones of the two halves next to
// 0x43 bytes, and one byte permute per dword assembles [q_2j, 0x43,
// q_2j+1, 0x43].
__device__ __forceinline__ u32x4 widen4(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;                                   // q0 q2 q4 q6
  const uint32_t h1 = (w >> 4) & 0x000F000Fu;                             // q1 . q5 .
  const uint32_t h3 = (w >> 12) & 0x000F000Fu;                            // q3 . q7 .
  const uint32_t a = h1 | 0x43004300u, b = h3 | 0x43004300u;
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(a, lo, 0x05040500u);   // q0 43 q1 43
  r[1] = __builtin_amdgcn_perm(b, lo, 0x05040501u);   // q2 43 q3 43
  r[2] = __builtin_amdgcn_perm(a, lo, 0x05060502u);   // q4 43 q5 43
  r[3] = __builtin_amdgcn_perm(b, lo, 0x05060503u);   // q6 43 q7 43
  return r;
}

// Eight 8-bit codes (two words, element i in byte i) as eight bf16 values q
// (integers below 256 are exact in bf16: the float's low 16 bits are zero).
__device__ __forceinline__ uint32_t widen8_pair(uint32_t w, int j) {
  const uint32_t a = __float_as_uint((float)((w >> (16 * j)) & 0xFFu));
  const uint32_t b = __float_as_uint((float)((w >> (16 * j + 8)) & 0xFFu));
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
__device__ __forceinline__ u32x4 widen8(u32x2 w) {
  return u32x4{widen8_pair(w[0], 0), widen8_pair(w[0], 1), widen8_pair(w[1], 0),
               widen8_pair(w[1], 1)};
}

__device__ __forceinline__ float bf16_at(const uint8_t* p) {
  return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
}

constexpr uint32_t kOnes = 0x3F803F80u;   // two bf16 1.0

struct QStreamParams {
  const uint16_t* a_src;        // GEMM 1: x [M, H]; GEMM 2: act [P, I]
  const uint8_t* wq;            // codes: GEMM 1 [E, 2I, H*bits/8]; GEMM 2 [E, H, I*bits/8]
  const uint8_t* sc;            // bf16 scales [rows, K/64]
  const uint8_t* bi;            // bf16 biases [rows, K/64]
  const int32_t* sorted;
  const int32_t* expert_ids;
  const int32_t* boff;
  const float* topk_weights;    // GEMM 2
  int M, top_k, E, H, I;
  uint16_t* out;                // GEMM 1: act [P, I]
  float* partial;               // GEMM 2: [P, H] fp32 weighted rows
};

// A tile is one block (16 pairs) and 128 weight rows: GEMM 1 the 64 gate
// rows f and the 64 up rows I + f of 64 act columns, GEMM 2 128 rows of W2.
// K streams in slices of 1024 / BITS elements, so every code row brings 128
// bytes (8 16-byte chunks, chunk c of row R at slot c ^ ((R >> 1) & 7):
// the 16 rows of an operand read fall on distinct banks) and a stage holds
// 16 KB of codes -- enough bytes in flight per workgroup to stream at HBM
// rate with two workgroups per CU.  Wave w owns two 16-row A tiles over the
// whole K (GEMM 1: gate rows 16w.. and up rows 64 + 16w..; GEMM 2: rows
// 32w.. and 32w + 16..), so no cross-wave reduction is needed; the pairs'
// rows (bf16 x or act) are the B operand.
constexpr int kWR = 128;                    // weight rows per tile
constexpr int kCRB = 128;                   // code bytes per row and slice
template <int BITS> constexpr int kslice() { return kCRB * 8 / BITS; }       // 256 / 128
template <int BITS> constexpr int groups() { return kslice<BITS>() / kGroup; }  // 4 / 2
template <int BITS> constexpr int arow_bytes() { return kslice<BITS>() * 2; }   // 512 / 256
constexpr int kAOff = kWR * kCRB;                                             // 16 KB
template <int BITS> constexpr int s_off() { return kAOff + kBM * arow_bytes<BITS>(); }
// scales then biases, [row][groups] bf16
template <int BITS> constexpr int sb_bytes() { return kWR * groups<BITS>() * 2; }
template <int BITS> constexpr int stage_bytes() { return s_off<BITS>() + 2 * sb_bytes<BITS>(); }
constexpr int kCodeCopies = kWR * kCRB / 1024 / kWaves;                        // 4
template <int BITS> constexpr int a_copies() { return kBM * arow_bytes<BITS>() / 1024 / kWaves; }
template <int BITS> constexpr int s_copies() { return 2 * sb_bytes<BITS>() / 256 / kWaves; }
template <int BITS> constexpr int copies() {
  return kCodeCopies + a_copies<BITS>() + s_copies<BITS>();
}
static_assert(stage_bytes<4>() * kStages * 2 + 256 <= 160 * 1024, "two workgroups per CU");
static_assert(a_copies<8>() == 1 && s_copies<8>() == 1 && a_copies<4>() == 2 &&
              s_copies<4>() == 2, "copy counts");

__device__ __forceinline__ int cslot(int R, int c) { return c ^ ((R >> 1) & 7); }
__device__ __forceinline__ int aslot(int R, int c) { return c ^ (R & 15); }

// kG1: GEMM 1 (x rows, SiLU(gate) * up into act) or GEMM 2 (act rows,
// weighted fp32 partial rows).
template <int BITS, bool kG1>
__global__ __launch_bounds__(kThreads, 2) void qgemm_stream_kernel(QStreamParams prm) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  __shared__ int s_pair[kBM];
  __shared__ float s_wt[kBM];
  constexpr int kSB = stage_bytes<BITS>();
  constexpr int kKS = kslice<BITS>();
  constexpr int kG = groups<BITS>();
  constexpr int kARB = arow_bytes<BITS>();
  constexpr int kAChunks = kARB / 16;                  // 32 / 16
  constexpr int kACopies = a_copies<BITS>();
  constexpr int kSCopies = s_copies<BITS>();

  const int P = prm.M * prm.top_k;
  const int H = prm.H, I = prm.I;
  const int K = kG1 ? H : I;                           // reduction length
  const int rowb = K * BITS / 8;                       // code bytes per weight row
  const int ng = K / kGroup;
  const int ntn = kG1 ? I / 64 : H / kWR;
  const int ntiles = prm.boff[prm.E] * ntn;
  const int nslice = ceil_div(K, kKS);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int T0 = kG1 ? 16 * wv : 32 * wv;              // this wave's two A tiles
  const int T1 = kG1 ? 64 + 16 * wv : 32 * wv + 16;

  const int chunk = ceil_div(ntiles, 8);
  const int xcd = blockIdx.x & 7, nslots = gridDim.x >> 3;
  const int tend = min(ntiles, (xcd + 1) * chunk);
  for (int t = xcd * chunk + (blockIdx.x >> 3); t < tend; t += nslots) {
    const int b = t / ntn, nt = t - b * ntn;
    wait_vmem<0>();
    const int e = prm.expert_ids[b];
    if (tid < kBM) {
      const int p = prm.sorted[b * kBM + tid];
      s_pair[tid] = p;
      if (!kG1) s_wt[tid] = p < P ? prm.topk_weights[p] : 0.f;
    }
    __syncthreads();

    // global weight row of tile row R
    auto wrow = [&](int R) -> size_t {
      if (kG1) return (size_t)e * 2 * I + (R < 64 ? 0 : I) + nt * 64 + (R & 63);
      return (size_t)e * H + nt * kWR + R;
    };
    const uint8_t* csrc[kCodeCopies];
    int cchunk[kCodeCopies];
#pragma unroll
    for (int i = 0; i < kCodeCopies; ++i) {
      const int R = (wv * kCodeCopies + i) * 8 + (lane >> 3);
      cchunk[i] = cslot(R, lane & 7);   // the slot map is its own inverse
      csrc[i] = prm.wq + wrow(R) * rowb;
    }
    const uint16_t* asrc[kACopies];
    int achunk[kACopies];
#pragma unroll
    for (int i = 0; i < kACopies; ++i) {
      const int R = (wv * kACopies + i) * (1024 / kARB) + lane / kAChunks;
      achunk[i] = aslot(R, lane % kAChunks);
      const int p = s_pair[R];
      asrc[i] = p >= P ? nullptr
                       : prm.a_src + (size_t)(kG1 ? p / prm.top_k : p) * K;
    }
    // scale / bias copies: flat dword j of the two [row][kG] arrays
    const uint8_t* ssrc[kSCopies];
    int sgrp[kSCopies];
#pragma unroll
    for (int i = 0; i < kSCopies; ++i) {
      const int j = (wv * kSCopies + i) * 64 + lane;
      const int arr = j / (kWR * kG / 2), jr = j - arr * (kWR * kG / 2);
      const int R = jr / (kG / 2), dw = jr - R * (kG / 2);
      sgrp[i] = dw * 2;
      ssrc[i] = (arr == 0 ? prm.sc : prm.bi) + wrow(R) * ng * 2;
    }

    auto issue = [&](int sl, int buf) {
      uint8_t* sb = ring + buf * kSB;
#pragma unroll
      for (int i = 0; i < kCodeCopies; ++i) {
        const int off = sl * kCRB + cchunk[i] * 16;
        load_lds16<kNonTemporal>(off < rowb ? (const void*)(csrc[i] + off) : (const void*)kZeroPage,
                                 sb + (wv * kCodeCopies + i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < kACopies; ++i) {
        const int k = sl * kKS + achunk[i] * 8;
        const bool ok = asrc[i] != nullptr && k < K;
        load_lds16(ok ? (const void*)(asrc[i] + k) : (const void*)kZeroPage,
                   sb + kAOff + (wv * kACopies + i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < kSCopies; ++i) {
        const int g = sl * kG + sgrp[i];
        copy_lds4(g < ng ? (const void*)(ssrc[i] + g * 2) : (const void*)kZeroPage,
                  sb + s_off<BITS>() + (wv * kSCopies + i) * 256);
      }
    };

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    const u32x4 ones = {kOnes, kOnes, kOnes, kOnes};
    issue(0, 0);
    if (nslice > 1) issue(1, 1);
    for (int sl = 0; sl < nslice; ++sl) {
      if (sl + 1 < nslice) wait_vmem<copies<BITS>()>(); else wait_vmem<0>();
      barrier_nofence();    // slice sl is in LDS; slice sl-1 has been consumed
      if (sl + 2 < nslice) issue(sl + 2, (sl + 2) % kStages);
      const uint8_t* sb = ring + (sl % kStages) * kSB;
      const uint8_t* ss = sb + s_off<BITS>();
      // every LDS read of the slice first (one round trip), then the math
      constexpr int kSteps = 2 * kG;                   // 32-element k steps
      using Codes = typename std::conditional<BITS == 4, uint32_t, u32x2>::type;
      u32x4 xb[kSteps];
      Codes c0[kSteps], c1[kSteps];
      const int R0 = T0 + r16, R1 = T1 + r16;
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) {
        xb[ks] = *reinterpret_cast<const u32x4*>(sb + kAOff + r16 * kARB +
                                                 (aslot(r16, ks * 4 + kg) << 4));
        // 4 bits: 32 codes = one 16-byte chunk per k step, dword kg is this
        // lane's 8; 8 bits: half chunk kg & 1 of chunk 2 ks + kg / 2
        const int c = BITS == 4 ? ks : ks * 2 + (kg >> 1);
        const int o = BITS == 4 ? kg * 4 : (kg & 1) * 8;
        c0[ks] = *reinterpret_cast<const Codes*>(sb + R0 * kCRB + (cslot(R0, c) << 4) + o);
        c1[ks] = *reinterpret_cast<const Codes*>(sb + R1 * kCRB + (cslot(R1, c) << 4) + o);
      }
      // scales and biases of rows 4 kg .. 4 kg + 3 of each A tile: 4 kG
      // consecutive bf16 values each ([row][kG] layout)
      constexpr int kSW = 2 * kG;                      // dwords per 4-row block
      uint32_t sw0[kSW], sw1[kSW], bw0[kSW], bw1[kSW];
#pragma unroll
      for (int i = 0; i < kSW; i += 4) {
        const int o0 = (T0 + 4 * kg) * kG * 2 + i * 4, o1 = (T1 + 4 * kg) * kG * 2 + i * 4;
        const u32x4 a = *reinterpret_cast<const u32x4*>(ss + o0);
        const u32x4 bq = *reinterpret_cast<const u32x4*>(ss + o1);
        const u32x4 c = *reinterpret_cast<const u32x4*>(ss + sb_bytes<BITS>() + o0);
        const u32x4 d = *reinterpret_cast<const u32x4*>(ss + sb_bytes<BITS>() + o1);
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          sw0[i + z] = a[z];
          sw1[i + z] = bq[z];
          bw0[i + z] = c[z];
          bw1[i + z] = d[z];
        }
      }
      auto half = [](const uint32_t* w, int idx) {
        return __uint_as_float(idx & 1 ? w[idx >> 1] & 0xFFFF0000u : w[idx >> 1] << 16);
      };
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = d0, dsx = d0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int ks = g * 2 + j;
          u32x4 a0, a1;
          if constexpr (BITS == 4) {
            a0 = widen4(c0[ks]);
            a1 = widen4(c1[ks]);
          } else {
            a0 = widen8(c0[ks]);
            a1 = widen8(c1[ks]);
          }
          d0 = mfma_16x16x32(a0, xb[ks], d0);
          d1 = mfma_16x16x32(a1, xb[ks], d1);
          dsx = mfma_16x16x32(ones, xb[ks], dsx);
        }
        // rows 4 kg + q of each A tile: acc += s D + (b [- 128 s]) S
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float s0 = half(sw0, q * kG + g), s1 = half(sw1, q * kG + g);
          float b0 = half(bw0, q * kG + g), b1 = half(bw1, q * kG + g);
          if constexpr (BITS == 4) {
            b0 -= 128.f * s0;
            b1 -= 128.f * s1;
          }
          acc0[q] = __builtin_fmaf(b0, dsx[q], __builtin_fmaf(s0, d0[q], acc0[q]));
          acc1[q] = __builtin_fmaf(b1, dsx[q], __builtin_fmaf(s1, d1[q], acc1[q]));
        }
      }
    }
    // lane holds rows 4 kg + q of each A tile for pair column r16
    const int p = s_pair[r16];
    if (p < P) {
      if constexpr (kG1) {
        u32x2 v;
        v[0] = pack_bf16x2(silu_mul(acc0[0], acc1[0]), silu_mul(acc0[1], acc1[1]));
        v[1] = pack_bf16x2(silu_mul(acc0[2], acc1[2]), silu_mul(acc0[3], acc1[3]));
        *reinterpret_cast<u32x2*>(prm.out + (size_t)p * I + nt * 64 + T0 + 4 * kg) = v;
      } else {
        float* dst = prm.partial + (size_t)p * H + nt * kWR + 4 * kg;
        *reinterpret_cast<f32x4*>(dst + T0) = s_wt[r16] * acc0;
        *reinterpret_cast<f32x4*>(dst + T1) = s_wt[r16] * acc1;
      }
    }
    __syncthreads();   // s_pair, s_wt and the ring are reused by the next tile
  }
}

long long persistent_grid(long long tiles) {
  long long grid = std::min<long long>(tiles, 2LL * moe_host::device_cu_count());
  return std::max<long long>(8, (grid + 7) / 8 * 8);
}

QStreamParams params(const moe_host::QGemmArgs& a) {
  QStreamParams prm{};
  prm.sorted = a.sorted_token_ids;
  prm.expert_ids = a.expert_ids;
  prm.boff = a.expert_block_offsets;
  prm.topk_weights = a.topk_weights;
  prm.M = a.M;
  prm.top_k = a.top_k;
  prm.E = a.E;
  prm.H = a.H;
  prm.I = a.I;
  prm.partial = a.partial;
  return prm;
}

template <int BITS>
hipError_t launch_q1(const moe_host::QGemmArgs& a, hipStream_t s) {
  QStreamParams prm = params(a);
  prm.a_src = a.x;
  prm.wq = reinterpret_cast<const uint8_t*>(a.w13q);
  prm.sc = reinterpret_cast<const uint8_t*>(a.w13_scales);
  prm.bi = reinterpret_cast<const uint8_t*>(a.w13_biases);
  prm.out = a.act;
  const long long grid = persistent_grid((long long)a.max_blocks * (a.I / 64));
  constexpr int kRing = kStages * stage_bytes<BITS>();
  static bool lds_set[moe_host::kMaxDevices] = {};
  const hipError_t err = moe_host::ensure_dynamic_lds(
      reinterpret_cast<const void*>(&qgemm_stream_kernel<BITS, true>), kRing, lds_set);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((qgemm_stream_kernel<BITS, true>), dim3((unsigned)grid), dim3(kThreads),
                     kRing, s, prm);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_q2(const moe_host::QGemmArgs& a, hipStream_t s) {
  QStreamParams prm = params(a);
  prm.a_src = a.act;
  prm.wq = reinterpret_cast<const uint8_t*>(a.w2q);
  prm.sc = reinterpret_cast<const uint8_t*>(a.w2_scales);
  prm.bi = reinterpret_cast<const uint8_t*>(a.w2_biases);
  const long long grid = persistent_grid((long long)a.max_blocks * (a.H / kWR));
  constexpr int kRing = kStages * stage_bytes<BITS>();
  static bool lds_set[moe_host::kMaxDevices] = {};
  hipError_t err = moe_host::ensure_dynamic_lds(
      reinterpret_cast<const void*>(&qgemm_stream_kernel<BITS, false>), kRing, lds_set);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((qgemm_stream_kernel<BITS, false>), dim3((unsigned)grid), dim3(kThreads),
                     kRing, s, prm);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return moe_host::launch_combine_partials(a.partial, a.M, a.top_k, a.H, a.out, s);
}

}  // namespace

namespace moe_host {

bool qgemm_stream_shapes_ok(int H, int I) { return H % 128 == 0 && I % 128 == 0; }

hipError_t launch_qgemm1_stream(const QGemmArgs& a, hipStream_t s) {
  return a.bits == 4 ? launch_q1<4>(a, s) : launch_q1<8>(a, s);
}

hipError_t launch_qgemm2_stream(const QGemmArgs& a, hipStream_t s) {
  return a.bits == 4 ? launch_q2<4>(a, s) : launch_q2<8>(a, s);
}

}  // namespace moe_host
