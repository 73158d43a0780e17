// Weight-streaming grouped GEMMs for small batches (about one pair per
// expert).  Page "Mixture of Experts in vLLM - From First Principles to
// fused_moe", sub-section "Each expert is now an ordinary GEMM": with n_e
// near 1 each expert reads all of its weights to make about one output row,
// so the cost is the weight bytes and the kernel's job is to stream them at
// full HBM bandwidth.
//
// Blocks of 16 pairs (index lists built with block_m = 16).  A tile is one
// block and 32 weight rows:
//   GEMM 1: 16 gate rows and the matching 16 up rows of W13[e] -> 16 act
//           columns (SiLU(gate) * up), rows p of act in pair order;
//   GEMM 2: 32 rows of W2[e] -> 32 output columns; the epilogue scales by
//           topk_weights[p], stores the fp32 partial row p, and the last of
//           the top_k producers of a (token, 32 columns) piece adds the
//           token's partial rows in slot order and writes bf16 (page
//           sections "Put the results back, and combine them per token" and
//           "The rest of the layer stays in pair order").
//
// Persistent workgroups (two per CU) walk the tiles; each XCD takes one
// contiguous range of tiles, so the tiles of one block (same gathered rows)
// run side by side under one L2.  Per tile, K is streamed through a 3-stage
// LDS ring of 256-element slices: one global_load_lds_dwordx4 of a wave
// copies 1 KB = two 512-byte row slices, weight rows with the non-temporal
// policy (they are read once).  In LDS, chunk c (16 bytes) of row R sits at
// slot c ^ (R & 15), which makes the 16-row MFMA operand reads
// conflict-free (measured).  The four waves split the eight 32-element k
// steps of a slice, accumulate 16x16x32 MFMA tiles (weights as A, the 16
// pair rows as B), and add their partial tiles through LDS at the end.
// Pads (id >= M*top_k), features past the end and the K tail copy a zeroed
// page.
#include <algorithm>

#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kBM = 16;                        // pairs per block
constexpr int kWRows = 32;                     // weight rows per tile
constexpr int kKS = 256;                       // k elements per slice
constexpr int kRowB = kKS * 2;                 // bytes per row slice
constexpr int kStages = 3;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kStageBytes = (kWRows + kBM) * kRowB;       // 24 KB
constexpr int kRingBytes = kStages * kStageBytes;          // 72 KB
constexpr int kWCopies = kWRows / 2 / kWaves;              // 1 KB copies per wave: weights (4)
constexpr int kXCopies = kBM / 2 / kWaves;                 //                       pair rows (2)
constexpr int kCopies = kWCopies + kXCopies;
// the reduction tiles and the output staging fit in one ring slot
static_assert(kWaves * 2 * 64 * 16 + kBM * (kWRows + 1) * 4 <= kStageBytes, "ring slot");

__device__ __forceinline__ int slot(int row, int chunk) { return chunk ^ (row & 15); }

struct StreamParams {
  const uint16_t* a_src;      // GEMM 1: x [M, H]; GEMM 2: act [P, I]
  const uint16_t* w;          // GEMM 1: w13 [E, 2I, H]; GEMM 2: w2 [E, H, I]
  const int32_t* sorted;
  const int32_t* expert_ids;
  const int32_t* boff;
  const float* topk_weights;  // GEMM 2
  int M, top_k, E, H, I;
  uint16_t* out;              // GEMM 1: act; GEMM 2: out [M, H]
  float* partial;             // GEMM 2: [P, H] fp32 weighted partial rows
  int32_t* counters;          // GEMM 2: [M, ceil(H / 32)] arrivals (zeroed)
};

template <bool kGemm1>
__global__ __launch_bounds__(kThreads, 2) void gemm_stream_kernel(StreamParams prm) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  __shared__ int s_pair[kBM];
  __shared__ float s_wt[kBM];
  __shared__ int s_last[kBM];

  const int P = prm.M * prm.top_k;
  const int K = kGemm1 ? prm.H : prm.I;
  const int ntn = kGemm1 ? ceil_div(prm.I, 16) : ceil_div(prm.H, kWRows);
  const int ntiles = prm.boff[prm.E] * ntn;
  const int nslice = ceil_div(K, kKS);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int half = lane >> 5, cl = lane & 31;          // copy: row in pair, chunk slot

  // XCD-contiguous persistent schedule (gridDim.x is a multiple of 8)
  const int chunk = ceil_div(ntiles, 8);
  const int xcd = blockIdx.x & 7, nslots = gridDim.x >> 3;
  const int tend = min(ntiles, (xcd + 1) * chunk);
  for (int t = xcd * chunk + (blockIdx.x >> 3); t < tend; t += nslots) {
    const int b = t / ntn, nt = t - b * ntn;
    wait_vmem<0>();   // the previous tile's stores are complete: only copies are counted below
    const int e = prm.expert_ids[b];
    if (tid < kBM) {
      const int p = prm.sorted[b * kBM + tid];
      s_pair[tid] = p;
      s_wt[tid] = (!kGemm1 && p < P) ? prm.topk_weights[p] : 0.f;
    }
    __syncthreads();

    // ---- this lane's copy sources: copy i of wave w moves rows 2(w*n+i), +1 ----
    const uint16_t* wsrc[kWCopies];
    int wchunk[kWCopies];
#pragma unroll
    for (int i = 0; i < kWCopies; ++i) {
      const int R = 2 * (wv * kWCopies + i) + half;
      wchunk[i] = cl ^ (R & 15);
      const uint16_t* row = nullptr;
      if (kGemm1) {
        const int f = nt * 16 + (R & 15);
        if (f < prm.I) row = prm.w + ((size_t)e * 2 * prm.I + (R < 16 ? f : prm.I + f)) * K;
      } else {
        const int h = nt * kWRows + R;
        if (h < prm.H) row = prm.w + ((size_t)e * prm.H + h) * K;
      }
      wsrc[i] = row;
    }
    const uint16_t* xsrc[kXCopies];
    int xchunk[kXCopies];
#pragma unroll
    for (int i = 0; i < kXCopies; ++i) {
      const int R = 2 * (wv * kXCopies + i) + half;
      xchunk[i] = cl ^ (R & 15);
      const int p = s_pair[R];
      const uint16_t* row = nullptr;
      if (p < P)
        row = kGemm1 ? prm.a_src + (size_t)(p / prm.top_k) * prm.H : prm.a_src + (size_t)p * prm.I;
      xsrc[i] = row;
    }
    auto issue = [&](int sl, int buf) {
      uint8_t* sb = ring + buf * kStageBytes;
#pragma unroll
      for (int i = 0; i < kWCopies; ++i) {
        const int k = sl * kKS + wchunk[i] * 8;
        const bool ok = wsrc[i] != nullptr && k < K;
        load_lds16<kNonTemporal>(ok ? (const void*)(wsrc[i] + k) : (const void*)kZeroPage,
                                 sb + (wv * kWCopies + i) * 2 * kRowB);
      }
#pragma unroll
      for (int i = 0; i < kXCopies; ++i) {
        const int k = sl * kKS + xchunk[i] * 8;
        const bool ok = xsrc[i] != nullptr && k < K;
        load_lds16(ok ? (const void*)(xsrc[i] + k) : (const void*)kZeroPage,
                   sb + (kWRows + (wv * kXCopies + i) * 2) * kRowB);
      }
    };

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    issue(0, 0);
    if (nslice > 1) issue(1, 1);
    for (int sl = 0; sl < nslice; ++sl) {
      if (sl + 1 < nslice) wait_vmem<kCopies>(); else wait_vmem<0>();
      barrier_nofence();    // slice sl is in LDS; slice sl-1 has been consumed
      if (sl + 2 < nslice) issue(sl + 2, (sl + 2) % kStages);
      const uint8_t* sb = ring + (sl % kStages) * kStageBytes;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = (wv * 2 + j) * 4 + kg;          // 16-byte chunk of the k step
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(sb + r16 * kRowB + (slot(r16, c) << 4));
        const u32x4 a1 =
            *reinterpret_cast<const u32x4*>(sb + (16 + r16) * kRowB + (slot(16 + r16, c) << 4));
        const u32x4 bx =
            *reinterpret_cast<const u32x4*>(sb + (kWRows + r16) * kRowB + (slot(r16, c) << 4));
        acc0 = mfma_16x16x32(a0, bx, acc0);
        acc1 = mfma_16x16x32(a1, bx, acc1);
      }
    }
    // The waves' partial tiles meet in the ring slot two slices behind the last
    // one: every wave has finished reading it (barrier of the last slice).
    f32x4(*red)[2][64] = reinterpret_cast<f32x4(*)[2][64]>(ring + (nslice % kStages) * kStageBytes);
    float(*s_ct)[kWRows + 1] = reinterpret_cast<float(*)[kWRows + 1]>(
        ring + (nslice % kStages) * kStageBytes + kWaves * 2 * 64 * sizeof(f32x4));
    red[wv][0][lane] = acc0;
    red[wv][1][lane] = acc1;
    __syncthreads();

    // lane holds rows 4 kg + q of each 16-row weight tile, for pair column r16
    if (kGemm1) {
      if (wv == 0) {
        f32x4 gs = red[0][0][lane], us = red[0][1][lane];
#pragma unroll
        for (int i = 1; i < kWaves; ++i) {
          gs += red[i][0][lane];
          us += red[i][1][lane];
        }
        const int p = s_pair[r16];
        const int nf = nt * 16 + 4 * kg;
        if (p < P && nf < prm.I) {
          u32x2 v;
          v[0] = pack_bf16x2(silu_mul(gs[0], us[0]), silu_mul(gs[1], us[1]));
          v[1] = pack_bf16x2(silu_mul(gs[2], us[2]), silu_mul(gs[3], us[3]));
          *reinterpret_cast<u32x2*>(prm.out + (size_t)p * prm.I + nf) = v;
        }
      }
      __syncthreads();   // red, s_pair and the ring are reused by the next tile
      continue;
    }

    // GEMM 2: sum the waves' tiles into s_ct[pair][column]
    if (wv < 2) {
      f32x4 v = red[0][wv][lane];
#pragma unroll
      for (int i = 1; i < kWaves; ++i) v += red[i][wv][lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) s_ct[r16][wv * 16 + 4 * kg + q] = v[q];
    }
    __syncthreads();
    // partial rows: thread -> (pair tid / 16, columns 2 (tid % 16), +1)
    const int H = prm.H;
    {
      const int pr = tid >> 4, c2 = (tid & 15) * 2;
      const int p = s_pair[pr];
      const int h = nt * kWRows + c2;
      if (p < P && h < H) {
        float* dst = prm.partial + (size_t)p * H + h;
        __hip_atomic_store(dst, s_wt[pr] * s_ct[pr][c2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(dst + 1, s_wt[pr] * s_ct[pr][c2 + 1], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // Every wave waits until its stores have completed; then one arrival per
    // (token, 32 columns).  The last of the top_k arrivals adds the token's
    // partial rows in slot order and writes the bf16 output piece.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int ncg = ceil_div(H, kWRows);
    if (tid < kBM) {
      const int p = s_pair[tid];
      int last = -1;
      if (p < P) {
        const int tok = p / prm.top_k;
        const int old = atomicAdd(prm.counters + (size_t)tok * ncg + nt, 1);
        if (old == prm.top_k - 1) last = tok;
      }
      s_last[tid] = last;
    }
    __syncthreads();
    for (int it = tid; it < kBM * kWRows; it += kThreads) {
      const int tok = s_last[it / kWRows];
      const int col = nt * kWRows + (it % kWRows);
      if (tok >= 0 && col < H)
        prm.out[(size_t)tok * H + col] = (uint16_t)f32_to_bf16(
            sum_partials(prm.partial + (size_t)tok * prm.top_k * H + col, H, prm.top_k));
    }
    __syncthreads();
  }
}

// GEMM 2 for small batches with register streaming: a workgroup owns one
// block and 64 rows of W2[e] (16 per wave, whole K per wave), loads weight
// and act rows straight into registers in the MFMA operand layout (four
// lanes of a row read 64 contiguous bytes per load), and runs the same
// combine epilogue with one arrival per (token, 64 columns).  With K = I
// (768 for the Qwen3 shape) a tile is too short for the LDS ring above to
// reach steady state, so this form is faster there.
constexpr int kSC = 256;   // k elements per register super-chunk (8 MFMA k steps)

__global__ __launch_bounds__(256) void gemm2_rows_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const float* __restrict__ topk_weights, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ expert_ids, const int32_t* __restrict__ boff, int M,
    int top_k, int E, int H, int I, uint16_t* __restrict__ out, float* __restrict__ partial,
    int32_t* __restrict__ counters) {
  __shared__ int s_last[kBM];
  __shared__ int s_pair[kBM];
  __shared__ float s_wt[kBM];
  __shared__ float ct[kBM][65];
  const int b = blockIdx.x;
  if (b >= boff[E]) return;
  const int P = M * top_k;
  const int e = expert_ids[b];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int h = blockIdx.y * 64 + wv * 16 + r;
  const bool h_ok = h < H;
  const uint16_t* wp = w2 + ((size_t)e * H + (h_ok ? h : 0)) * I;
  const int p = sorted[b * kBM + r];
  const bool p_ok = p < P;
  const uint16_t* ap = act + (size_t)(p_ok ? p : 0) * I;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nsc = ceil_div(I, kSC);
  for (int sc = 0; sc < nsc; ++sc) {
    const int kb = sc * kSC + g * 8;
    u32x4 wa[8], ab[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int k = kb + s * 32;
      const bool kin = k < I;
      wa[s] = load16_or_zero(wp + k, h_ok && kin);
      ab[s] = load16_or_zero(ap + k, p_ok && kin);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma_16x16x32(wa[s], ab[s], acc);
  }

  // lane holds output columns blockIdx.y*64 + wv*16 + 4g + q of pair r.
  // The workgroup's 64-column x 16-pair tile goes through LDS so that each
  // store instruction writes 64 consecutive columns of one partial row
  // (row p = topk_weights[p] * (W2[e] act[p]), fp32, agent-coherent stores).
  ct[r][wv * 16 + 4 * g + 0] = acc[0];
  ct[r][wv * 16 + 4 * g + 1] = acc[1];
  ct[r][wv * 16 + 4 * g + 2] = acc[2];
  ct[r][wv * 16 + 4 * g + 3] = acc[3];
  if (threadIdx.x < kBM) {
    const int pp = sorted[b * kBM + threadIdx.x];
    s_pair[threadIdx.x] = pp;
    s_wt[threadIdx.x] = pp < P ? topk_weights[pp] : 0.f;
  }
  __syncthreads();
  const int hc = blockIdx.y * 64 + lane;
  if (hc < H) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pr = wv * 4 + i;
      const int pp = s_pair[pr];
      if (pp >= P) continue;
      __hip_atomic_store(partial + (size_t)pp * H + hc, s_wt[pr] * ct[pr][lane], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // Every wave waits until its stores have completed, then the workgroup
  // counts one arrival per (token, 64 columns).  The last of the top_k
  // arrivals adds the token's top_k partial rows in slot order (coherent
  // loads) and writes the bf16 output piece.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int ncg = ceil_div(H, 64);
  if (threadIdx.x < kBM) {
    const int pr = s_pair[threadIdx.x];
    int last = -1;
    if (pr < P) {
      const int t = pr / top_k;
      const int old = atomicAdd(counters + (size_t)t * ncg + blockIdx.y, 1);
      if (old == top_k - 1) last = t;
    }
    s_last[threadIdx.x] = last;
  }
  __syncthreads();
  for (int it = wv; it < kBM; it += 4) {
    const int t = s_last[it];
    if (t < 0) continue;
    if (hc < H)
      out[(size_t)t * H + hc] =
          (uint16_t)f32_to_bf16(sum_partials(partial + (size_t)t * top_k * H + hc, H, top_k));
  }
}


template <bool kGemm1>
hipError_t launch_stream(const moe_host::GemmArgs& a, hipStream_t s) {
  StreamParams prm;
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
  prm.out = a.out;
  prm.partial = a.partial;
  prm.counters = a.counters;
  // persistent grid: two workgroups per CU at most, never more than the tiles
  const long long ntn = kGemm1 ? (a.I + 15) / 16 : (a.H + kWRows - 1) / kWRows;
  const long long tiles = (long long)a.max_blocks * ntn;
  long long grid = std::min<long long>(tiles, 2LL * moe_host::device_cu_count());
  grid = std::max<long long>(8, (grid + 7) / 8 * 8);
  static bool attr_set = false;   // idempotent; racing first calls set the same value
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_stream_kernel<kGemm1>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kRingBytes);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL((gemm_stream_kernel<kGemm1>), dim3((unsigned)grid), dim3(kThreads),
                     kRingBytes, s, prm);
  return hipGetLastError();
}

}  // namespace

namespace moe_host {

hipError_t launch_gemm1_stream(const GemmArgs& a, hipStream_t s) { return launch_stream<true>(a, s); }

hipError_t launch_gemm2_stream(const GemmArgs& a, hipStream_t s) {
  dim3 grid(a.max_blocks, ceil_div_host(a.H, 64));
  hipLaunchKernelGGL(gemm2_rows_kernel, grid, dim3(256), 0, s, a.a_src, a.w, a.topk_weights,
                     a.sorted_token_ids, a.expert_ids, a.expert_block_offsets, a.M, a.top_k, a.E,
                     a.H, a.I, a.out, a.partial, a.counters);
  return hipGetLastError();
}

}  // namespace moe_host
