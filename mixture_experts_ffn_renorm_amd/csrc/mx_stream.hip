// MXFP8 GEMM 1 for small batches (block_m 16) with the GEMM 2 input
// quantizer in its epilogue.  Page "Mixture of Experts in vLLM - From First
// Principles to fused_moe", sub-sections "One GEMM 1 program, step by step"
// (one block of pairs against one expert's gate and up rows, SiLU(gate) * up
// fused) and "The two index lists" (the FP8 GEMM inputs are quantized
// copies); the format is MXFP8 (OCP microscaling: per 32 consecutive k one
// E8M0 scale, E4M3 elements), named in the MLX part of the page "SGLang
// issue #22283".
//
// A tile is one block of 16 pairs and 32 act columns: the 32 gate rows f and
// the 32 up rows I + f of W13[e], so a tile's act row of one pair is exactly
// one 32-value MX block, and the epilogue quantizes it in place of a separate
// launch: act = bf16(SiLU(gate) * up) (the value the bf16 layer stores),
// shared exponent floor(log2 amax) - 8 over the 32 values, each value
// rounded to the nearest E4M3 of v / 2^shared (ties to even, saturated);
// codes and scale byte go straight to the GEMM 2 input.
//
// K (= H bytes of E4M3) streams in 256-byte slices -- two steps of the
// gfx950 scaled MFMA 16x16x128 -- through a 3-stage LDS ring filled by
// global_load_lds: 64 weight rows (16 KB, non-temporal) and the 16 gathered
// x code rows per stage, plus a 4-byte copy per lane of the rows' scale
// bytes for the slice; row R's 16-byte chunk c sits at slot c ^ (R & 15).
// Wave w owns one 16-row A tile (gate columns 0..15, 16..31, then the
// matching up rows) over the whole K; the operand layout of the scaled MFMA
// (lane (r, g) supplies chunks g and 4 + g of a 128-k step and the scale
// byte of block g of its row) is the one the other MXFP8 kernels use.
// Persistent workgroups, two per CU, each XCD walking one contiguous range
// of tiles.  Pads, the K tail and rows past the tile copy the zeroed page.
#include <algorithm>

#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kBM = 16;
constexpr int kWRows = 64;                         // 32 gate + 32 up rows
constexpr int kKS = 256;                           // bytes (= k) per row slice
constexpr int kStages = 3;
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kXOff = kWRows * kKS;                // 16 KB of weights
constexpr int kSOff = kXOff + kBM * kKS;           // + 4 KB of x codes
constexpr int kStageBytes = kSOff + kWaves * 256;  // + 8 scale bytes x 128 rows (80 used)
constexpr int kWCopies = kWRows * kKS / 1024 / kWaves;   // 4 (1 KB = 4 rows)
constexpr int kCopies = kWCopies + 2;                    // + x rows + scales
static_assert(kWaves * 64 * 16 <= kStageBytes, "reduction area");

__device__ __forceinline__ int slot(int R, int c) { return c ^ (R & 15); }

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

__device__ __forceinline__ float bf16_round(float v) { return __uint_as_float(f32_to_bf16(v) << 16); }

struct MxqParams {
  const uint8_t* x;          // x codes [M, H]
  const uint8_t* xs;         // x scales [M, H/32]
  const uint8_t* w;          // W13 codes [E, 2I, H]
  const uint8_t* ws;         // W13 scales [E, 2I, H/32]
  const int32_t* sorted;
  const int32_t* expert_ids;
  const int32_t* boff;
  int M, top_k, E, H, I;
  uint8_t* qact;             // act codes [P, I]
  uint8_t* sact;             // act scales [P, I/32]
};

__global__ __launch_bounds__(kThreads, 2) void gemm1_stream_mxq_kernel(MxqParams prm) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  __shared__ int s_pair[kBM];
  const int P = prm.M * prm.top_k;
  const int H = prm.H, I = prm.I, nb = H / 32;
  const int ntn = I / 32;
  const int ntiles = prm.boff[prm.E] * ntn;
  const int nslice = ceil_div(H, kKS);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int crow = lane >> 4, cl = lane & 15;      // copy: row within the 4, slot

  const int chunk = ceil_div(ntiles, 8);
  const int xcd = blockIdx.x & 7, nslots = gridDim.x >> 3;
  const int tend = min(ntiles, (xcd + 1) * chunk);
  for (int t = xcd * chunk + (blockIdx.x >> 3); t < tend; t += nslots) {
    const int b = t / ntn, nt = t - b * ntn;
    wait_vmem<0>();   // the previous tile's stores are complete: only copies are counted below
    const int e = prm.expert_ids[b];
    if (tid < kBM) s_pair[tid] = prm.sorted[b * kBM + tid];
    __syncthreads();

    // tile row R: gate row nt*32 + R (R < 32) or up row I + nt*32 + R - 32
    auto wrow = [&](int R) -> size_t {
      return (size_t)e * 2 * I + (R < 32 ? 0 : I) + nt * 32 + (R & 31);
    };
    const uint8_t* wsrc[kWCopies];
    int wch[kWCopies];
#pragma unroll
    for (int i = 0; i < kWCopies; ++i) {
      const int R = (wv * kWCopies + i) * 4 + crow;
      wch[i] = slot(R, cl);   // the slot map is its own inverse
      wsrc[i] = prm.w + wrow(R) * H;
    }
    const int xr = wv * 4 + crow;
    const int xp = s_pair[xr];
    const uint8_t* xsrc = xp < P ? prm.x + (size_t)(xp / prm.top_k) * H : nullptr;
    const int xch = slot(xr, cl);
    // dword sj of the scale area: row sj / 2 (0..63 weights, 64..79 x rows,
    // others none), blocks 8 sl + 4 (sj & 1) .. + 3 of the slice
    const int sj = wv * 64 + lane, srow = sj >> 1, sdw = sj & 1;
    const uint8_t* ssrc = nullptr;
    if (srow < kWRows) {
      ssrc = prm.ws + wrow(srow) * nb;
    } else if (srow < kWRows + kBM) {
      const int p = s_pair[srow - kWRows];
      if (p < P) ssrc = prm.xs + (size_t)(p / prm.top_k) * nb;
    }

    auto issue = [&](int sl, int buf) {
      uint8_t* sb = ring + buf * kStageBytes;
#pragma unroll
      for (int i = 0; i < kWCopies; ++i) {
        const int off = sl * kKS + wch[i] * 16;
        load_lds16<kNonTemporal>(off < H ? (const void*)(wsrc[i] + off) : (const void*)kZeroPage,
                                 sb + (wv * kWCopies + i) * 1024);
      }
      const int xo = sl * kKS + xch * 16;
      load_lds16((xsrc != nullptr && xo < H) ? (const void*)(xsrc + xo) : (const void*)kZeroPage,
                 sb + kXOff + wv * 1024);
      const int blk = sl * 8 + sdw * 4;   // H % 128 == 0: a dword's 4 blocks are all in or all out
      copy_lds4((ssrc != nullptr && blk < nb) ? (const void*)(ssrc + blk) : (const void*)kZeroPage,
                sb + kSOff + wv * 256);
    };

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int Ra = wv * 16 + r16;
    issue(0, 0);
    if (nslice > 1) issue(1, 1);
    for (int sl = 0; sl < nslice; ++sl) {
      if (sl + 1 < nslice) wait_vmem<kCopies>(); else wait_vmem<0>();
      barrier_nofence();    // slice sl is in LDS; slice sl-1 has been consumed
      if (sl + 2 < nslice) issue(sl + 2, (sl + 2) % kStages);
      const uint8_t* sb = ring + (sl % kStages) * kStageBytes;
      const uint8_t* sc = sb + kSOff;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int c0 = st * 8 + kg, c1 = c0 + 4;
        const i32x8 a = cat_u32x4(
            *reinterpret_cast<const u32x4*>(sb + Ra * kKS + (slot(Ra, c0) << 4)),
            *reinterpret_cast<const u32x4*>(sb + Ra * kKS + (slot(Ra, c1) << 4)));
        const i32x8 bx = cat_u32x4(
            *reinterpret_cast<const u32x4*>(sb + kXOff + r16 * kKS + (slot(r16, c0) << 4)),
            *reinterpret_cast<const u32x4*>(sb + kXOff + r16 * kKS + (slot(r16, c1) << 4)));
        const int blk = st * 4 + kg;
        acc = mfma_mx(a, bx, acc, sc[Ra * 8 + blk], sc[(kWRows + r16) * 8 + blk]);
      }
    }

    // Epilogue.  The four waves' tiles meet in the ring slot two slices
    // behind the last one (every wave has passed the last slice's barrier);
    // lane (r16, kg) of wave w holds rows 4 kg + q of A tile w for pair r16.
    f32x4(*red)[64] = reinterpret_cast<f32x4(*)[64]>(ring + (nslice % kStages) * kStageBytes);
    red[wv][lane] = acc;
    __syncthreads();
    {
      // thread: pair pr, act columns 2j and 2j + 1 of the tile's 32
      const int pr = tid >> 4, j = tid & 15;
      const int c = j >> 3, within = (2 * j) & 15, kq = within >> 2, q = within & 3;
      const f32x4 g = red[c][kq * 16 + pr], u = red[2 + c][kq * 16 + pr];
      const float v0 = bf16_round(silu_mul(g[q], u[q]));
      const float v1 = bf16_round(silu_mul(g[q + 1], u[q + 1]));
      float amax = __builtin_fmaxf(__builtin_fabsf(v0), __builtin_fabsf(v1));
      amax = row16_max(amax);   // the 16 threads of pair pr are one DPP row
      const int shared = mx_shared_exp(amax);
      const int p = s_pair[pr];
      if (p < P) {
        const uint32_t code = e4m3_of(v0, shared) | (e4m3_of(v1, shared) << 8);
        *reinterpret_cast<uint16_t*>(prm.qact + (size_t)p * I + nt * 32 + 2 * j) = (uint16_t)code;
        if (j == 0) prm.sact[(size_t)p * (I / 32) + nt] = (uint8_t)(shared + 127);
      }
    }
    __syncthreads();   // red, s_pair and the ring are reused by the next tile
  }
}

}  // namespace

namespace moe_host {

hipError_t launch_gemm1_stream_mx_quantize(const GemmArgs& a, uint8_t* qact, uint8_t* sact,
                                           hipStream_t s) {
  MxqParams prm{};
  prm.x = reinterpret_cast<const uint8_t*>(a.a_src);
  prm.xs = a.a_scales;
  prm.w = reinterpret_cast<const uint8_t*>(a.w);
  prm.ws = a.w_scales;
  prm.sorted = a.sorted_token_ids;
  prm.expert_ids = a.expert_ids;
  prm.boff = a.expert_block_offsets;
  prm.M = a.M;
  prm.top_k = a.top_k;
  prm.E = a.E;
  prm.H = a.H;
  prm.I = a.I;
  prm.qact = qact;
  prm.sact = sact;
  const long long tiles = (long long)a.max_blocks * (a.I / 32);
  long long grid = std::min<long long>(tiles, 2LL * device_cu_count());
  grid = std::max<long long>(8, (grid + 7) / 8 * 8);
  constexpr int kRing = kStages * kStageBytes;
  hipLaunchKernelGGL(gemm1_stream_mxq_kernel, dim3((unsigned)grid), dim3(kThreads), kRing, s, prm);
  return hipGetLastError();
}

}  // namespace moe_host
