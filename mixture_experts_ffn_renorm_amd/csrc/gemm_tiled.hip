// LDS-tiled MFMA grouped GEMMs for batches with many pairs per expert.
//
// GEMM 1 (page "Mixture of Experts in vLLM - From First Principles to
// fused_moe", sub-section "One GEMM 1 program, step by step"): a workgroup
// owns one block of BM pairs (one expert, from the index lists) and 128
// columns of the activation.  It reads expert_ids[b], skips pad entries
// (id >= M*top_k), reads input row p // top_k of x in place, multiplies by
// the matching 128 gate rows and 128 up rows of W13[e], and writes
// SiLU(gate) * up to row p of act (sub-section "The rest of the layer stays
// in pair order"), so the [M*top_k, 2I] product never reaches memory.
//
// GEMM 2 (same page, "The rest of the layer stays in pair order" and "Put
// the results back, and combine them per token"): the same tiling over
// act (row p read directly) and 256 rows of W2[e]; the epilogue scales row p
// by topk_weights[p] and stores it as an fp32 partial row p; the last of the
// top_k workgroups that produce a (token, 64-column group) adds that
// token's top_k partial rows in slot order and writes the bf16 output row
// piece in token order (no separate sum kernel, no atomic adds on data).
//
// Tile: 256 weight rows x BM pairs x 64 k per stage, 8 waves in a 4 x 2
// layout, each wave 64 weight rows x BM/2 pairs of 16x16x32 bf16 MFMAs.
// Weights are the MFMA A operand and pairs the B operand, so each lane ends
// with 4 consecutive features of one pair.
//
// Memory pipeline: operands go from global memory straight into LDS with
// global_load_lds_dwordx4 (no register staging), three stages deep.  One
// load instruction of a wave fills 1 KB of LDS = 8 rows of 64 k values; a
// row's eight 16-byte chunks are stored XOR-swizzled (chunk c of row R at
// slot c ^ ((R >> 1) & 7)), so the 16 rows that one MFMA operand read
// touches fall on distinct banks, while each global access still reads
// whole 128-byte row pieces.  Rows or k ranges outside the operands (pads,
// features past the end, the K tail) load from a zeroed 16-byte page.
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kBK = 64;          // k elements per stage = 128 bytes per row
constexpr int kBN = 256;         // weight rows per tile
constexpr int kStages = 3;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowBytes = kBK * 2;

template <int BM>
struct TileCfg {
  static constexpr int kWGroups = kBN / 8 / kWaves;   // 8-row W groups per wave (4)
  static constexpr int kXGroups = BM / 8 / kWaves;    // 8-row X groups per wave (2 or 1)
  static constexpr int kLoads = kWGroups + kXGroups;  // load instructions per stage
  static constexpr int kStageBytes = (kBN + BM) * kRowBytes;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kNT = BM / 32;                 // 16-pair MFMA tiles per wave
};

// Slot of a row's 16-byte chunk: chunk c of row R sits at c ^ swz(R).  With
// this choice the 16 rows read by one MFMA operand load (same chunk, rows
// R0..R0+15) hit distinct LDS banks on gfx950 (measured: the same
// ds_read_b128 throughput as contiguous reads; a 144-byte padded row
// stride, or the XOR with (R ^ (R >> 3)) & 7, both run at about half).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

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
  float* partial;      // GEMM 2: [M*top_k, H] fp32 weighted partial rows
  int32_t* counters;
};

template <int BM, bool kGemm1>
__global__ __launch_bounds__(kThreads, 1) void gemm_tiled_kernel(TileParams prm) {
  using C = TileCfg<BM>;
  constexpr int NT = C::kNT;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int s_pair[BM];
  __shared__ float s_wt[BM];
  __shared__ int s_last[4 * BM];

  const int P = prm.M * prm.top_k;
  const int nblocks = prm.boff[prm.E];
  const int tile = xcd_contiguous_tile(blockIdx.x, nblocks * prm.ntiles_n);
  if (tile < 0) return;
  const int b = tile / prm.ntiles_n;
  const int nt = tile - b * prm.ntiles_n;
  const int e = prm.expert_ids[b];
  const int K = kGemm1 ? prm.H : prm.I;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  if (tid < BM) {
    const int p = prm.sorted[b * BM + tid];
    s_pair[tid] = p;
    s_wt[tid] = (!kGemm1 && p < P) ? prm.topk_weights[p] : 0.f;
  }

  // ---- per-lane source row of each load slot (row R of the LDS tile) ----
  const int lrow = lane >> 3, lpos = lane & 7;
  const uint16_t* wsrc[C::kWGroups];
  int wchunk[C::kWGroups];
#pragma unroll
  for (int i = 0; i < C::kWGroups; ++i) {
    const int R = (wv + kWaves * i) * 8 + lrow;
    wchunk[i] = lpos ^ swz(R);
    const uint16_t* row = nullptr;
    if (kGemm1) {
      const int f = nt * 128 + (R & 127);
      if (f < prm.I)
        row = prm.w + ((size_t)e * 2 * prm.I + (R < 128 ? f : prm.I + f)) * K;
    } else {
      const int h = nt * kBN + R;
      if (h < prm.H) row = prm.w + ((size_t)e * prm.H + h) * K;
    }
    wsrc[i] = row;
  }
  const uint16_t* xsrc[C::kXGroups];
  int xchunk[C::kXGroups];
#pragma unroll
  for (int i = 0; i < C::kXGroups; ++i) {
    const int R = (wv + kWaves * i) * 8 + lrow;
    xchunk[i] = lpos ^ swz(R);
    const int p = prm.sorted[b * BM + R];
    const uint16_t* row = nullptr;
    if (p < P)
      row = kGemm1 ? prm.a_src + (size_t)(p / prm.top_k) * prm.H
                   : prm.a_src + (size_t)p * prm.I;
    xsrc[i] = row;
  }

  auto issue_stage = [&](int kt, int buf) {
    uint8_t* sb = lds + buf * C::kStageBytes;
#pragma unroll
    for (int i = 0; i < C::kWGroups; ++i) {
      const int k = kt * kBK + wchunk[i] * 8;
      const void* src = (wsrc[i] != nullptr && k < K) ? (const void*)(wsrc[i] + k)
                                                      : (const void*)kZeroPage;
      load_lds16(src, sb + (wv + kWaves * i) * 8 * kRowBytes);
    }
#pragma unroll
    for (int i = 0; i < C::kXGroups; ++i) {
      const int k = kt * kBK + xchunk[i] * 8;
      const void* src = (xsrc[i] != nullptr && k < K) ? (const void*)(xsrc[i] + k)
                                                      : (const void*)kZeroPage;
      load_lds16(src, sb + (kBN + (wv + kWaves * i) * 8) * kRowBytes);
    }
  };

  // ---- this wave's MFMA tiles ----
  const int wf = wv & 3, wp = wv >> 2;
  int arow[4];
  if (kGemm1) {
    arow[0] = wf * 32;        arow[1] = wf * 32 + 16;         // gate rows
    arow[2] = 128 + wf * 32;  arow[3] = 128 + wf * 32 + 16;   // matching up rows
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) arow[i] = wf * 64 + 16 * i;
  }
  const int brow0 = wp * (BM / 2);
  const int r16 = lane & 15, kg = lane >> 4;
  // byte offsets inside a stage of this lane's operand reads, per k half s
  int aoff[2][4], boffs[2][NT];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int c = s * 4 + kg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int R = arow[i] + r16;
      aoff[s][i] = R * kRowBytes + ((c ^ swz(R)) << 4);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int R = brow0 + 16 * j + r16;
      boffs[s][j] = (kBN + R) * kRowBytes + ((c ^ swz(R)) << 4);
    }
  }

  f32x4 acc[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = ceil_div(K, kBK);
  issue_stage(0, 0);
  if (nk > 1) issue_stage(1, 1);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once at most the next stage's loads are pending
    if (kt + 1 < nk) wait_vmem<C::kLoads>(); else wait_vmem<0>();
    // Every wave's part of stage kt is in LDS, and stage kt-1 is consumed.
    barrier_nofence();
    if (kt + 2 < nk) issue_stage(kt + 2, (kt + 2) % kStages);
    const uint8_t* sb = lds + (kt % kStages) * C::kStageBytes;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 af[4], bfr[NT];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const u32x4*>(sb + aoff[s][i]);
#pragma unroll
      for (int j = 0; j < NT; ++j) bfr[j] = *reinterpret_cast<const u32x4*>(sb + boffs[s][j]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma_16x16x32(af[i], bfr[j], acc[i][j]);
    }
  }

  // ---- epilogues: lane holds features 4*kg + q of each A tile, pair r16 of each B tile ----
  if (kGemm1) {
    const int I = prm.I;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int p = s_pair[brow0 + 16 * j + r16];
      if (p >= P) continue;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = nt * 128 + wf * 32 + 16 * i + 4 * kg;
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

  // GEMM 2: the wave's 64 x BM/2 tile goes through LDS so that each store
  // instruction writes 64 consecutive columns of one partial row.  Row p of
  // the fp32 partials holds topk_weights[p] * (W2[e] act[p]); the stores are
  // agent-coherent, so other workgroups' coherent loads see them once they
  // have completed.
  const int H = prm.H;
  constexpr int kCt = 65;                           // row stride in floats
  __syncthreads();                                  // all waves done reading the stages
  float* ct = reinterpret_cast<float*>(lds) + wv * (BM / 2) * kCt;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) ct[(16 * j + r16) * kCt + 16 * i + 4 * kg + q] = acc[i][j][q];
  __builtin_amdgcn_wave_barrier();
  const int h = nt * kBN + wf * 64 + lane;
  if (h < H) {
    for (int pr = 0; pr < BM / 2; ++pr) {
      const int p = s_pair[brow0 + pr];
      if (p >= P) continue;
      __hip_atomic_store(prm.partial + (size_t)p * H + h, s_wt[brow0 + pr] * ct[pr * kCt + lane],
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // The last arrival per (token, 64-column group) sums the token's top_k
  // partial rows in slot order and writes the bf16 result.  Every wave first
  // waits until its own stores have completed; the workgroup then counts
  // its arrivals (4 column groups per tile).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int ncg = ceil_div(H, 64);
  for (int it = tid; it < 4 * BM; it += kThreads) {
    const int r = it % BM, cgl = it / BM;
    const int cg = nt * 4 + cgl;
    const int p = s_pair[r];
    int last = -1;
    if (p < P && cg < ncg) {
      const int t = p / prm.top_k;
      const int old = atomicAdd(prm.counters + (size_t)t * ncg + cg, 1);
      if (old == prm.top_k - 1) last = t;
    }
    s_last[it] = last;
  }
  __syncthreads();
  for (int it = wv; it < 4 * BM; it += kWaves) {
    const int t = s_last[it];
    if (t < 0) continue;
    const int col = (nt * 4 + it / BM) * 64 + lane;
    if (col < H)
      prm.out[(size_t)t * H + col] =
          (uint16_t)f32_to_bf16(sum_partials(prm.partial + (size_t)t * prm.top_k * H + col, H,
                                             prm.top_k));
  }
}

// the GEMM 2 epilogue reuses the stage LDS for 8 waves x (BM/2) x 65 floats
static_assert(TileCfg<64>::kLdsBytes >= kWaves * 32 * 65 * 4, "epilogue LDS");
static_assert(TileCfg<128>::kLdsBytes >= kWaves * 64 * 65 * 4, "epilogue LDS");

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
  prm.ntiles_n = kGemm1 ? moe_host::ceil_div_host(a.I, 128) : moe_host::ceil_div_host(a.H, kBN);
  prm.out = a.out;
  prm.partial = a.partial;
  prm.counters = a.counters;
  const long long tiles = (long long)a.max_blocks * prm.ntiles_n;
  const unsigned grid = (unsigned)(((tiles + 7) / 8) * 8);
  const size_t lds = TileCfg<BM>::kLdsBytes;
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
