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
//   GEMM 2: 64 rows of W2[e] -> 64 output columns; the epilogue scales by
//           topk_weights[p] and stores the fp32 partial row p, and a second
//           small kernel adds each token's top_k partial rows in slot order
//           and writes bf16 (page sections "The rest of the layer stays in
//           pair order" and "Put the results back, and combine them per
//           token"); see the GEMM 2 notes below.
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
//
// MXFP8 operands (kMX; E4M3 bytes, one E8M0 scale per 32 k): the same row
// slices hold twice the k values, and a wave's two 32-k bf16 steps become
// one step of the gfx950 scaled MFMA 16x16x128, whose lane (r, g) operand
// is the two 16-byte chunks g and 4 + g of a 128-k piece -- the chunks the
// bf16 form reads for its two steps -- with the scale of k block g of its
// row.  Each slice also copies the rows' scale bytes for its k range into
// a small LDS area (4-byte copies, one per lane of every wave; rows past
// the tile and blocks past K read the zeroed page).
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
constexpr int kWCopies = kWRows / 2 / kWaves;              // 1 KB copies per wave: weights (4)
constexpr int kXCopies = kBM / 2 / kWaves;                 //                       pair rows (2)
constexpr int kCopies = kWCopies + kXCopies;
// MX: 16 scale bytes per row per slice (512 k), 48 rows, copied 4 bytes per
// lane by all four waves (1 KB of LDS per stage)
constexpr int kScaleBytes = kWaves * 64 * 4;
template <bool kMX>
constexpr int stage_bytes() { return kStageBytes + (kMX ? kScaleBytes : 0); }
// the waves' partial tiles fit in one ring slot
static_assert(kWaves * 2 * 64 * 16 <= kStageBytes, "ring slot");

__device__ __forceinline__ int slot(int row, int chunk) { return chunk ^ (row & 15); }

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8 cat_u32x4(u32x4 lo, u32x4 hi) {
  const u32x4 l = lo, h = hi;   // by value
  return i32x8{(int)l[0], (int)l[1], (int)l[2], (int)l[3], (int)h[0], (int)h[1], (int)h[2], (int)h[3]};
}

// D = A B + C over 128 k of E4M3 operands, each lane's 32 values scaled by
// 2^(its E8M0 byte - 127).
__device__ __forceinline__ f32x4 mfma_mx(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ void copy_lds4(const void* src, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)lds_dst, 4, 0, 0);
}

struct StreamParams {
  const uint16_t* a_src;      // GEMM 1: x [M, H]; GEMM 2: act [P, I]  (MX: E4M3 bytes)
  const uint16_t* w;          // GEMM 1: w13 [E, 2I, H]; GEMM 2: w2 [E, H, I]
  const uint8_t* a_scales;    // MX: E8M0 per 32 k of each a_src row
  const uint8_t* w_scales;    // MX: E8M0 per 32 k of each weight row
  const int32_t* sorted;
  const int32_t* expert_ids;
  const int32_t* boff;
  const float* topk_weights;  // GEMM 2
  int M, top_k, E, H, I;
  uint16_t* out;              // GEMM 1: act; GEMM 2: out [M, H]
  float* partial;             // GEMM 2: [P, H] fp32 weighted partial rows
};

template <bool kMX>
__global__ __launch_bounds__(kThreads, 2) void gemm1_stream_kernel(StreamParams prm) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  __shared__ int s_pair[kBM];
  constexpr int kSB = stage_bytes<kMX>();

  const int P = prm.M * prm.top_k;
  const int K = kMX ? prm.H / 2 : prm.H;   // row length in 2-byte units (MX: H % 128 == 0)
  const int nb = prm.H / 32;               // MX: scale bytes per row
  const int ntn = ceil_div(prm.I, 16);
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
    if (tid < kBM) s_pair[tid] = prm.sorted[b * kBM + tid];
    __syncthreads();

    // ---- this lane's copy sources: copy i of wave w moves rows 2(w*n+i), +1 ----
    const uint16_t* wsrc[kWCopies];
    int wchunk[kWCopies];
#pragma unroll
    for (int i = 0; i < kWCopies; ++i) {
      const int R = 2 * (wv * kWCopies + i) + half;
      wchunk[i] = cl ^ (R & 15);
      const int f = nt * 16 + (R & 15);
      wsrc[i] = f < prm.I ? prm.w + ((size_t)e * 2 * prm.I + (R < 16 ? f : prm.I + f)) * K : nullptr;
    }
    const uint16_t* xsrc[kXCopies];
    int xchunk[kXCopies];
#pragma unroll
    for (int i = 0; i < kXCopies; ++i) {
      const int R = 2 * (wv * kXCopies + i) + half;
      xchunk[i] = cl ^ (R & 15);
      const int p = s_pair[R];
      xsrc[i] = p < P ? prm.a_src + (size_t)(p / prm.top_k) * K : nullptr;
    }
    // MX: lane q = 64 wv + lane copies dword q % 4 of row q / 4's 16 scale
    // bytes of a slice (rows: 32 weight rows, 16 pair rows, then none)
    const uint8_t* ssrc = nullptr;
    const int sq = wv * 64 + lane, srow = sq >> 2, sdw = sq & 3;
    if constexpr (kMX) {
      if (srow < kWRows) {
        const int f = nt * 16 + (srow & 15);
        if (f < prm.I)
          ssrc = prm.w_scales + ((size_t)e * 2 * prm.I + (srow < 16 ? f : prm.I + f)) * nb;
      } else if (srow < kWRows + kBM) {
        const int p = s_pair[srow - kWRows];
        if (p < P) ssrc = prm.a_scales + (size_t)(p / prm.top_k) * nb;
      }
    }
    auto issue = [&](int sl, int buf) {
      uint8_t* sb = ring + buf * kSB;
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
      if constexpr (kMX) {
        const int blk = sl * 16 + sdw * 4;        // first of this dword's 4 blocks
        const bool ok = ssrc != nullptr && blk < nb;
        copy_lds4(ok ? (const void*)(ssrc + blk) : (const void*)kZeroPage,
                  sb + kStageBytes + wv * 256);
      }
    };

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    issue(0, 0);
    if (nslice > 1) issue(1, 1);
    for (int sl = 0; sl < nslice; ++sl) {
      if (sl + 1 < nslice) wait_vmem<kCopies + (kMX ? 1 : 0)>(); else wait_vmem<0>();
      barrier_nofence();    // slice sl is in LDS; slice sl-1 has been consumed
      if (sl + 2 < nslice) issue(sl + 2, (sl + 2) % kStages);
      const uint8_t* sb = ring + (sl % kStages) * kSB;
      if constexpr (kMX) {
        // chunks 8 wv + kg and 8 wv + 4 + kg: k block 4 wv + kg of the slice
        const int c0 = wv * 8 + kg, c1 = c0 + 4;
        const uint8_t* sc = sb + kStageBytes;
        const i32x8 a0 = cat_u32x4(
            *reinterpret_cast<const u32x4*>(sb + r16 * kRowB + (slot(r16, c0) << 4)),
            *reinterpret_cast<const u32x4*>(sb + r16 * kRowB + (slot(r16, c1) << 4)));
        const i32x8 a1 = cat_u32x4(
            *reinterpret_cast<const u32x4*>(sb + (16 + r16) * kRowB + (slot(16 + r16, c0) << 4)),
            *reinterpret_cast<const u32x4*>(sb + (16 + r16) * kRowB + (slot(16 + r16, c1) << 4)));
        const i32x8 bx = cat_u32x4(
            *reinterpret_cast<const u32x4*>(sb + (kWRows + r16) * kRowB + (slot(r16, c0) << 4)),
            *reinterpret_cast<const u32x4*>(sb + (kWRows + r16) * kRowB + (slot(r16, c1) << 4)));
        const int blk = wv * 4 + kg;
        const int s0 = sc[r16 * 16 + blk], s1 = sc[(16 + r16) * 16 + blk];
        const int sx = sc[(kWRows + r16) * 16 + blk];
        acc0 = mfma_mx(a0, bx, acc0, s0, sx);
        acc1 = mfma_mx(a1, bx, acc1, s1, sx);
        continue;
      }
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
    f32x4(*red)[2][64] = reinterpret_cast<f32x4(*)[2][64]>(ring + (nslice % kStages) * kSB);
    red[wv][0][lane] = acc0;
    red[wv][1][lane] = acc1;
    __syncthreads();

    // lane holds rows 4 kg + q of each 16-row weight tile, for pair column r16
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
  }
}

// GEMM 2 for small batches, streamed through LDS like GEMM 1 but organised
// for its short K (= I): a tile is one block and 64 rows of W2[e] (one
// 16-row MFMA tile per wave, whole K per wave, so no cross-wave reduction),
// K slices are 128 elements (256-byte row slices, chunk c of row R at slot
// c ^ (R & 15), measured conflict-free), and each persistent workgroup owns
// a contiguous range of tiles.  Consecutive tiles of one block share the
// expert and the gathered act rows, so the copy ring keeps streaming across
// tile boundaries and a tile's combine epilogue runs while the next tile's
// first slices are in flight; the ring is drained only where the block
// changes.  Epilogue: each lane stores its four columns of the tile (64
// columns x 16 pairs) straight from its MFMA registers as fp32 partial rows
// p = topk_weights[p] * (W2[e] act[p]) -- no LDS staging and no barrier, so
// the next slices' copies keep streaming.  (Measured at 64 tokens: the
// kernel runs ~67 us against ~59 us for the same ring streaming the same
// bytes with no compute; dropping the 4 MB of partial-row stores recovers
// ~5 us, while LDS staging, barriers, deferring the stores to the end of
// the run, and streaming across block boundaries changed nothing.)  The
// per-token sum is the small combine kernel below (at these batch sizes the
// partial rows are a few MB, while an in-kernel last-arrival combine costs
// each tile three serialized memory round trips).
namespace ring2 {

constexpr int kBM = 16;
constexpr int kWRows = 64;
constexpr int kKS = 128;
constexpr int kRowB = kKS * 2;                              // 256 bytes
constexpr int kStages = 3;
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kStageBytes = (kWRows + kBM) * kRowB;         // 20 KB
constexpr int kWCopies = kWRows / 4 / kWaves;               // 1 KB = 4 rows; per wave (4)
constexpr int kXCopies = kBM / 4 / kWaves;                  // (1)
constexpr int kCopies = kWCopies + kXCopies;
// MX: 8 scale bytes per row per slice (256 k), 80 rows, copied 4 bytes per
// lane by all four waves (1 KB of LDS per stage)
constexpr int kScaleBytes = kWaves * 64 * 4;
template <bool kMX>
constexpr int stage_bytes() { return kStageBytes + (kMX ? kScaleBytes : 0); }

__device__ __forceinline__ int slot(int row, int chunk) { return chunk ^ (row & 15); }

template <bool kMX>
__global__ __launch_bounds__(kThreads, 2) void gemm2_ring_kernel(StreamParams prm) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  __shared__ int s_pair[kBM];
  __shared__ float s_wt[kBM];
  __shared__ int s_e;
  constexpr int kSB = stage_bytes<kMX>();

  const int P = prm.M * prm.top_k;
  const int H = prm.H, K = kMX ? prm.I / 2 : prm.I;   // 2-byte units (MX: I % 128 == 0)
  const int nb = prm.I / 32;                         // MX: scale bytes per row
  const int ntn = ceil_div(H, kWRows);
  const int ntiles = prm.boff[prm.E] * ntn;
  const int ns = ceil_div(K, kKS);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int crow = lane >> 4, cl = lane & 15;       // copy: row within the 4, chunk slot

  // contiguous range of tiles per workgroup inside its XCD's range
  const int xcd = blockIdx.x & 7, nslots = gridDim.x >> 3, myslot = blockIdx.x >> 3;
  const int chunk = ceil_div(ntiles, 8);
  const int xbeg = xcd * chunk, xend = min(ntiles, xbeg + chunk);
  const int per = ceil_div(max(xend - xbeg, 0), nslots);
  int t = xbeg + myslot * per;
  const int tstop = min(xend, t + per);

  while (t < tstop) {
    const int b = t / ntn;
    const int run_end = min(tstop, (b + 1) * ntn);   // my tiles of block b: t .. run_end-1
    wait_vmem<0>();
    if (tid < kBM) {
      const int p = prm.sorted[b * kBM + tid];
      s_pair[tid] = p;
      s_wt[tid] = p < P ? prm.topk_weights[p] : 0.f;
    }
    if (tid == kBM) s_e = prm.expert_ids[b];
    __syncthreads();
    const int e = s_e;
    const uint16_t* wbase = prm.w + (size_t)e * H * K;
    // gathered act rows: copy of wave w moves rows 4 w .. 4 w + 3
    const int xr = wv * 4 + crow;
    const int xp = s_pair[xr];
    const uint16_t* xsrc = xp < P ? prm.a_src + (size_t)xp * K : nullptr;
    const int xchunk = cl ^ (xr & 15);
    const int nt0 = t - b * ntn;
    const int G = (run_end - t) * ns;                 // slices of this run
    // MX: lane q = 64 wv + lane copies dword q % 2 of row q / 2's 8 scale
    // bytes of a slice (rows: 64 weight rows, 16 pair rows, then none)
    const int sq = wv * 64 + lane, srow = sq >> 1, sdw = sq & 1;
    const uint8_t* sx_src = nullptr;
    if constexpr (kMX) {
      if (srow >= kWRows && srow < kWRows + kBM) {
        const int p = s_pair[srow - kWRows];
        if (p < P) sx_src = prm.a_scales + (size_t)p * nb;
      }
    }

    auto issue = [&](int g) {
      const int nt = nt0 + g / ns, sl = g - (g / ns) * ns;
      uint8_t* sb = ring + (g % kStages) * kSB;
#pragma unroll
      for (int i = 0; i < kWCopies; ++i) {
        const int R = (wv * kWCopies + i) * 4 + crow;
        const int h = nt * kWRows + R;
        const int k = sl * kKS + (cl ^ (R & 15)) * 8;
        const bool ok = h < H && k < K;
        load_lds16<kNonTemporal>(ok ? (const void*)(wbase + (size_t)h * K + k) : (const void*)kZeroPage,
                                 sb + (wv * kWCopies + i) * 4 * kRowB);
      }
      const int k = sl * kKS + xchunk * 8;
      load_lds16((xsrc != nullptr && k < K) ? (const void*)(xsrc + k) : (const void*)kZeroPage,
                 sb + (kWRows + wv * 4) * kRowB);
      if constexpr (kMX) {
        const int blk = sl * 8 + sdw * 4;          // first of this dword's 4 blocks
        const uint8_t* src = nullptr;
        if (srow < kWRows) {
          const int h = nt * kWRows + srow;
          if (h < H) src = prm.w_scales + ((size_t)e * H + h) * nb;
        } else {
          src = sx_src;
        }
        const bool ok = src != nullptr && blk < nb;
        copy_lds4(ok ? (const void*)(src + blk) : (const void*)kZeroPage, sb + kStageBytes + wv * 256);
      }
    };

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    issue(0);
    if (G > 1) issue(1);
    for (int g = 0; g < G; ++g) {
      if (g + 1 < G) wait_vmem<kCopies + (kMX ? 1 : 0)>(); else wait_vmem<0>();
      barrier_nofence();    // slice g is in LDS; slice g-1 has been consumed
      if (g + 2 < G) issue(g + 2);
      const uint8_t* sb = ring + (g % kStages) * kSB;
      if constexpr (kMX) {
        // two 128-k steps per slice: chunks 8 s + kg and 8 s + 4 + kg, block 4 s + kg
        const uint8_t* sc = sb + kStageBytes;
        const int Ra = wv * 16 + r16;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int c0 = st * 8 + kg, c1 = c0 + 4;
          const i32x8 a = cat_u32x4(
              *reinterpret_cast<const u32x4*>(sb + Ra * kRowB + (slot(Ra, c0) << 4)),
              *reinterpret_cast<const u32x4*>(sb + Ra * kRowB + (slot(Ra, c1) << 4)));
          const i32x8 bx = cat_u32x4(
              *reinterpret_cast<const u32x4*>(sb + (kWRows + r16) * kRowB + (slot(r16, c0) << 4)),
              *reinterpret_cast<const u32x4*>(sb + (kWRows + r16) * kRowB + (slot(r16, c1) << 4)));
          const int blk = st * 4 + kg;
          acc = mfma_mx(a, bx, acc, sc[Ra * 8 + blk], sc[(kWRows + r16) * 8 + blk]);
        }
      } else {
#pragma unroll
      for (int j = 0; j < kKS / 32; ++j) {
        const int c = j * 4 + kg;
        const int Ra = wv * 16 + r16;
        const u32x4 a = *reinterpret_cast<const u32x4*>(sb + Ra * kRowB + (slot(Ra, c) << 4));
        const u32x4 bx =
            *reinterpret_cast<const u32x4*>(sb + (kWRows + r16) * kRowB + (slot(r16, c) << 4));
        acc = mfma_16x16x32(a, bx, acc);
      }
      }
      if (g % ns != ns - 1) continue;

      // ---- tile epilogue, straight from registers (no LDS, no barrier; the
      //      copies of the next slices stay in flight): lane holds rows
      //      wv*16 + 4 kg + q (q = 0..3) of the tile for pair column r16 ----
      const int nt = nt0 + g / ns;
      const int p = s_pair[r16];
      const int h = nt * kWRows + wv * 16 + 4 * kg;   // H % 8 == 0: all four exist or none
      if (p < P && h < H)
        *reinterpret_cast<f32x4*>(prm.partial + (size_t)p * H + h) = s_wt[r16] * acc;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    t = run_end;
    __syncthreads();                   // s_pair / s_e are reloaded for the next block
  }
}

// out[t, h] = bf16(sum over slots j of partial[t*top_k + j, h]), j ascending.
// Page "Mixture of Experts in vLLM ...", section "Put the results back, and
// combine them per token".  Thread: 4 consecutive columns of one token; all
// top_k loads are issued before the first add (one memory round trip, not
// top_k of them).
__global__ __launch_bounds__(256) void combine_partials_kernel(const float* __restrict__ partial,
                                                               int M, int top_k, int H,
                                                               uint16_t* __restrict__ out) {
  constexpr int kMaxK = 32;
  const int h4 = H / 4;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)M * h4) return;
  const int t = (int)(i / h4), h = (int)(i - (long long)t * h4) * 4;
  const float* src = partial + (size_t)t * top_k * H + h;
  f32x4 part[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < top_k) part[j] = *reinterpret_cast<const f32x4*>(src + (size_t)j * H);
  f32x4 sum = part[0];
#pragma unroll
  for (int j = 1; j < kMaxK; ++j)
    if (j < top_k) sum += part[j];
  u32x2 v;
  v[0] = pack_bf16x2(sum[0], sum[1]);
  v[1] = pack_bf16x2(sum[2], sum[3]);
  *reinterpret_cast<u32x2*>(out + (size_t)t * H + h) = v;
}

}  // namespace ring2

template <bool kMX>
hipError_t launch_gemm1(const moe_host::GemmArgs& a, hipStream_t s) {
  StreamParams prm{};
  prm.a_src = a.a_src;
  prm.w = a.w;
  prm.a_scales = a.a_scales;
  prm.w_scales = a.w_scales;
  prm.sorted = a.sorted_token_ids;
  prm.expert_ids = a.expert_ids;
  prm.boff = a.expert_block_offsets;
  prm.M = a.M;
  prm.top_k = a.top_k;
  prm.E = a.E;
  prm.H = a.H;
  prm.I = a.I;
  prm.out = a.out;
  // persistent grid: two workgroups per CU at most, never more than the tiles
  const long long tiles = (long long)a.max_blocks * ((a.I + 15) / 16);
  long long grid = std::min<long long>(tiles, 2LL * moe_host::device_cu_count());
  grid = std::max<long long>(8, (grid + 7) / 8 * 8);
  constexpr int kRing = kStages * stage_bytes<kMX>();
  static bool lds_set[moe_host::kMaxDevices] = {};
  const hipError_t err = moe_host::ensure_dynamic_lds(
      reinterpret_cast<const void*>(&gemm1_stream_kernel<kMX>), kRing, lds_set);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gemm1_stream_kernel<kMX>, dim3((unsigned)grid), dim3(kThreads), kRing, s, prm);
  return hipGetLastError();
}

template <bool kMX>
hipError_t launch_gemm2(const moe_host::GemmArgs& a, hipStream_t s) {
  StreamParams prm{};
  prm.a_src = a.a_src;
  prm.w = a.w;
  prm.a_scales = a.a_scales;
  prm.w_scales = a.w_scales;
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
  const long long tiles = (long long)a.max_blocks * ((a.H + ring2::kWRows - 1) / ring2::kWRows);
  long long grid = std::min<long long>(tiles, 2LL * moe_host::device_cu_count());
  grid = std::max<long long>(8, (grid + 7) / 8 * 8);
  constexpr int kRing = ring2::kStages * ring2::stage_bytes<kMX>();
  static bool lds_set[moe_host::kMaxDevices] = {};
  hipError_t err = moe_host::ensure_dynamic_lds(
      reinterpret_cast<const void*>(&ring2::gemm2_ring_kernel<kMX>), kRing, lds_set);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(ring2::gemm2_ring_kernel<kMX>, dim3((unsigned)grid), dim3(ring2::kThreads),
                     kRing, s, prm);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return moe_host::launch_combine_partials(a.partial, a.M, a.top_k, a.H, a.out, s);
}

}  // namespace

namespace moe_host {

hipError_t launch_gemm1_stream(const GemmArgs& a, hipStream_t s) {
  return a.mx ? launch_gemm1<true>(a, s) : launch_gemm1<false>(a, s);
}

hipError_t launch_gemm2_stream(const GemmArgs& a, hipStream_t s) {
  return a.mx ? launch_gemm2<true>(a, s) : launch_gemm2<false>(a, s);
}

hipError_t launch_combine_partials(const float* partial, int M, int top_k, int H, uint16_t* out,
                                   hipStream_t s) {
  const long long n4 = (long long)M * (H / 4);
  hipLaunchKernelGGL(ring2::combine_partials_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256),
                     0, s, partial, M, top_k, H, out);
  return hipGetLastError();
}

}  // namespace moe_host
