// LDS-tiled MFMA grouped GEMMs for batches with many pairs per expert.
//
// GEMM 1 (page "Mixture of Experts in vLLM - From First Principles to
// fused_moe", sub-section "One GEMM 1 program, step by step"): a workgroup
// owns one block of BM pairs (one expert, from the index lists) and 64
// columns of the activation.  It reads expert_ids[b], masks pad entries
// (id >= M*top_k), reads input row p // top_k of x in place, multiplies by
// the matching 64 gate rows and 64 up rows of W13[e], and writes
// SiLU(gate) * up to row p of act (sub-section "The rest of the layer stays
// in pair order"), so the [M*top_k, 2I] product never reaches memory.
//
// GEMM 2 (same page, "The rest of the layer stays in pair order" and "Put
// the results back, and combine them per token"): the same tiling over
// act (row p read directly) and W2[e]; the epilogue scales row p by
// topk_weights[p] and adds it into an fp32 per-token sum; the last of the
// top_k contributions to a (token, 64-column group) converts that group to
// bf16 in token order, so the [M*top_k, H] product never reaches memory.
//
// Tile: 128 weight rows x BM pairs x 64 k, 4 waves in a 2 x 2 layout, each
// wave 64 weight rows x BM/2 pairs of 16x16x32 bf16 MFMAs.  Operands are
// staged through double-buffered LDS with a 16-byte row pad (row stride
// 144 B keeps the 16 rows of one MFMA operand read on distinct banks).
// Weights are the MFMA A operand and pairs the B operand, so each lane ends
// with 4 consecutive features of one pair (8-byte bf16 stores for act).
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kBK = 64;
constexpr int kLdsStride = kBK + 8;   // elements per LDS row
constexpr int kWRows = 128;           // weight rows per tile
constexpr int kThreads = 256;

template <int BM>
constexpr size_t lds_bytes() {
  return (size_t)2 * (kWRows + BM) * kLdsStride * sizeof(uint16_t);
}

struct TileParams {
  const uint16_t* a_src;
  const uint16_t* w;
  const int32_t* sorted;
  const int32_t* expert_ids;
  const int32_t* boff;
  const float* topk_weights;
  int M, top_k, E, H, I;
  int ntiles_n;        // feature tiles per block
  uint16_t* out;
  float* acc;
  int32_t* counters;
};

template <int BM, bool kGemm1>
__global__ __launch_bounds__(kThreads, 2) void gemm_tiled_kernel(TileParams prm) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  constexpr int NT = BM / 32;                // 16-pair tiles per wave
  constexpr int XR = BM / 32;                // pair rows loaded per thread
  uint16_t* Ws = lds;                                   // [2][128][72]
  uint16_t* Xs = lds + 2 * kWRows * kLdsStride;         // [2][BM][72]

  const int P = prm.M * prm.top_k;
  const int nblocks = prm.boff[prm.E];
  const int tile = xcd_contiguous_tile(blockIdx.x, nblocks * prm.ntiles_n);
  if (tile < 0) return;
  const int b = tile / prm.ntiles_n;
  const int nt = tile - b * prm.ntiles_n;
  const int e = prm.expert_ids[b];
  const int K = kGemm1 ? prm.H : prm.I;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wf = wv & 1, wp = wv >> 1;

  // ---- per-thread global row pointers (chunk c of rows rg + 32 i) ----
  const int c = tid & 7, rg = tid >> 3;
  const uint16_t* wptr[4];
  const uint16_t* xptr[XR];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = rg + 32 * i;
    if (kGemm1) {
      const int n0 = nt * 64;
      const int f = r < 64 ? n0 + r : n0 + (r - 64);
      const bool ok = f < prm.I;
      const size_t row = (size_t)e * 2 * prm.I + (r < 64 ? f : prm.I + f);
      wptr[i] = ok ? prm.w + row * K : nullptr;
    } else {
      const int h = nt * 128 + r;
      wptr[i] = h < prm.H ? prm.w + ((size_t)e * prm.H + h) * K : nullptr;
    }
  }
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int p = prm.sorted[b * BM + rg + 32 * i];
    if (p < P)
      xptr[i] = kGemm1 ? prm.a_src + (size_t)(p / prm.top_k) * prm.H
                       : prm.a_src + (size_t)p * prm.I;
    else
      xptr[i] = nullptr;
  }

  u32x4 wreg[4], xreg[XR];
  auto gload = [&](int kt) {
    const int k = kt * kBK + c * 8;
    const bool kin = k < K;
#pragma unroll
    for (int i = 0; i < 4; ++i) wreg[i] = load16_or_zero(wptr[i] + k, wptr[i] != nullptr && kin);
#pragma unroll
    for (int i = 0; i < XR; ++i) xreg[i] = load16_or_zero(xptr[i] + k, xptr[i] != nullptr && kin);
  };
  auto lstore = [&](int buf) {
    uint16_t* wb = Ws + buf * kWRows * kLdsStride;
    uint16_t* xb = Xs + buf * BM * kLdsStride;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(wb + (rg + 32 * i) * kLdsStride + c * 8) = wreg[i];
#pragma unroll
    for (int i = 0; i < XR; ++i)
      *reinterpret_cast<u32x4*>(xb + (rg + 32 * i) * kLdsStride + c * 8) = xreg[i];
  };

  // A tiles (weight rows in the LDS tile) of this wave
  int arow[4];
  if (kGemm1) {
    arow[0] = wf * 32;       arow[1] = wf * 32 + 16;        // gate
    arow[2] = 64 + wf * 32;  arow[3] = 64 + wf * 32 + 16;   // matching up rows
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) arow[i] = wf * 64 + 16 * i;
  }
  const int brow0 = wp * (BM / 2);
  const int r16 = lane & 15, kg = lane >> 4;

  f32x4 acc[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = ceil_div(K, kBK);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t* wb = Ws + cur * kWRows * kLdsStride;
    const uint16_t* xb = Xs + cur * BM * kLdsStride;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kof = s * 32 + kg * 8;
      u32x4 af[4], bfr[NT];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(wb + (arow[i] + r16) * kLdsStride + kof);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bfr[j] = *reinterpret_cast<const u32x4*>(xb + (brow0 + 16 * j + r16) * kLdsStride + kof);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma_16x16x32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogues: lane holds features 4*kg + q of each A tile, pair r16 of each B tile ----
  if (kGemm1) {
    const int I = prm.I;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int p = prm.sorted[b * BM + brow0 + 16 * j + r16];
      if (p >= P) continue;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = nt * 64 + wf * 32 + 16 * i + 4 * kg;
        if (n >= I) continue;
        const f32x4 gt = acc[i][j], up = acc[i + 2][j];
        u32x2 v;
        v[0] = pack_bf16x2(silu_mul(gt[0], up[0]), silu_mul(gt[1], up[1]));
        v[1] = pack_bf16x2(silu_mul(gt[2], up[2]), silu_mul(gt[3], up[3]));
        *reinterpret_cast<u32x2*>(prm.out + (size_t)p * I + n) = v;
      }
    }
    return;
  }

  const int H = prm.H;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int p = prm.sorted[b * BM + brow0 + 16 * j + r16];
    if (p >= P) continue;
    const int t = p / prm.top_k;
    const float wt = prm.topk_weights[p];
    float* dst = prm.acc + (size_t)t * H;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = nt * 128 + wf * 64 + 16 * i + 4 * kg;
      if (h >= H) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) unsafeAtomicAdd(dst + h + q, wt * acc[i][j][q]);
    }
  }

  // ---- last arrival per (token, 64-column group) writes the bf16 row piece.
  // Every wave waits until its additions are performed, then the workgroup
  // counts its arrivals; the last of the top_k arrivals reads the finished
  // sums with atomic exchanges (served where the additions were performed;
  // they also leave the sums at zero).
  __shared__ int s_last[2 * BM];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int ncg = ceil_div(H, 64);
  if (tid < 2 * BM) {
    const int r = tid % BM, cgl = tid / BM;
    const int cg = nt * 2 + cgl;
    const int p = prm.sorted[b * BM + r];
    int last = -1;
    if (p < P && cg < ncg) {
      const int t = p / prm.top_k;
      const int old = atomicAdd(prm.counters + (size_t)t * ncg + cg, 1);
      if (old == prm.top_k - 1) last = t;
    }
    s_last[tid] = last;
  }
  __syncthreads();
  for (int it = wv; it < 2 * BM; it += 4) {
    const int t = s_last[it];
    if (t < 0) continue;
    const int col = (nt * 2 + it / BM) * 64 + lane;
    if (col < H) {
      const float v = atomicExch(prm.acc + (size_t)t * H + col, 0.0f);
      prm.out[(size_t)t * H + col] = (uint16_t)f32_to_bf16(v);
    }
  }
}

template <int BM, bool kGemm1>
hipError_t launch_tiled(const moe_host::GemmArgs& a, hipStream_t s) {
  TileParams prm;
  prm.a_src = a.a_src;
  prm.w = a.w;
  prm.sorted = a.sorted_token_ids;
  prm.expert_ids = a.expert_ids;
  prm.boff = a.expert_block_offsets;
  prm.topk_weights = a.topk_weights;
  prm.M = a.M;
  prm.top_k = a.top_k;
  prm.E = a.E;
  prm.H = a.H;
  prm.I = a.I;
  prm.ntiles_n = kGemm1 ? moe_host::ceil_div_host(a.I, 64) : moe_host::ceil_div_host(a.H, 128);
  prm.out = a.out;
  prm.acc = a.acc;
  prm.counters = a.counters;
  const long long tiles = (long long)a.max_blocks * prm.ntiles_n;
  const unsigned grid = (unsigned)(((tiles + 7) / 8) * 8);
  const size_t lds = lds_bytes<BM>();
  static bool attr_set = false;   // idempotent; racing first calls set the same value
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_tiled_kernel<BM, kGemm1>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL((gemm_tiled_kernel<BM, kGemm1>), dim3(grid), dim3(kThreads), lds, s, prm);
  return hipGetLastError();
}

}  // namespace

namespace moe_host {

hipError_t launch_gemm1_tiled(const GemmArgs& a, hipStream_t s) {
  if (a.block_m == 128) return launch_tiled<128, true>(a, s);
  return launch_tiled<64, true>(a, s);
}

hipError_t launch_gemm2_tiled(const GemmArgs& a, hipStream_t s) {
  if (a.block_m == 128) return launch_tiled<128, false>(a, s);
  return launch_tiled<64, false>(a, s);
}

}  // namespace moe_host
