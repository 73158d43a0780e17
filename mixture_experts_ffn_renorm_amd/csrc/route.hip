// Router: logits = W_r x (MFMA, fp32 accumulate), then per token softmax
// over all experts, ordered top-k (exact ties -> lower id) and renormalize.
// Page "Mixture of Experts in vLLM - From First Principles to fused_moe",
// section "One expert, and one token", sub-section "One token uses only 8
// experts".
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kTokTile = 16;     // tokens per MFMA tile (B columns)

// Router logits on the matrix cores, logits[t, e] = sum_h x[t, h] W_r[e, h]
// (+ bias[e]), fp32 accumulation of exact bf16 products.  W_r rows are the
// A operand, token rows the B operand; lane l (row/column r = l % 16, group
// g = l / 16) loads elements k0 + 8 g .. + 7 of its row for the 32-element
// k step at k0, so the four lanes of a row read 64 contiguous bytes.
//
// Small batches: a workgroup owns 16 tokens x 16 experts and its 4 waves
// split K in four contiguous ranges; partial tiles are added through LDS.
// Many workgroups read W_r in parallel.
// grid: (ceil(M / 16), ceil(E / 16)); block: 256.
__global__ __launch_bounds__(256) void route_logits_small_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int M, int H, int E, float* __restrict__ logits,
    float* __restrict__ zero_ptr, size_t zero_words) {
  // Optional clearing of counters used by kernels that follow on the same
  // stream.
  if (zero_ptr != nullptr) {
    const size_t nwg = (size_t)gridDim.x * gridDim.y;
    const size_t wg = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    const size_t n4 = zero_words >> 2;
    u32x4 z = {0u, 0u, 0u, 0u};
    for (size_t i = wg * 256 + threadIdx.x; i < n4; i += nwg * 256)
      reinterpret_cast<u32x4*>(zero_ptr)[i] = z;
    for (size_t i = (n4 << 2) + wg * 256 + threadIdx.x; i < zero_words; i += nwg * 256)
      zero_ptr[i] = 0.0f;
  }
  __shared__ f32x4 red[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * kTokTile;
  const int e0 = blockIdx.y * 16;
  const int erow = e0 + r, trow = t0 + r;
  const bool e_ok = erow < E, t_ok = trow < M;
  const uint16_t* ap = wr + (size_t)(e_ok ? erow : 0) * H;
  const uint16_t* bp = x + (size_t)(t_ok ? trow : 0) * H;
  const int kw = ceil_div(ceil_div(H, 4), 32) * 32;
  const int kbeg = min(H, w * kw);
  const int kend = min(H, kbeg + kw);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 16;   // k steps whose loads are in flight together
  for (int k0 = kbeg; k0 < kend; k0 += 32 * U) {
    u32x4 av[U], bv[U];
#pragma unroll
    for (int s = 0; s < U; ++s) {
      const int k = k0 + 32 * s + 8 * g;
      const bool kin = k < kend;   // kend is H or a multiple of 32; H % 8 == 0
      av[s] = load16_or_zero(ap + k, e_ok && kin);
      bv[s] = load16_or_zero(bp + k, t_ok && kin);
    }
#pragma unroll
    for (int s = 0; s < U; ++s) acc = mfma_16x16x32(av[s], bv[s], acc);
  }
  red[w][lane] = acc;
  __syncthreads();
  if (w != 0) return;
  acc = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
  // C: lane holds experts e0 + 4g + q (q = 0..3) for token t0 + r.
  if (t_ok) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + 4 * g + q;
      if (e < E) {
        float v = acc[q];
        if (bias != nullptr) v += bias[e];
        logits[(size_t)trow * E + e] = v;
      }
    }
  }
}

// Router logits for very small batches (M <= 16), GEMV-style: wave w of
// workgroup (bx, by) owns expert e = 4 bx + w and tokens 4 by .. 4 by + 3.
// Lane l takes the 16-byte chunks l, l + 64, ... of the W_r row and of the
// token rows (NC per lane per pass of 512 NC elements), all loads of a pass
// in flight together; fp32 products of the exact bf16 values, one wave sum
// per token.  Many workgroups (one per 4 experts) read W_r at once.
constexpr int kGemvTokens = 4;

template <int NC>
__global__ __launch_bounds__(256) void route_logits_gemv_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int M, int H, int E, float* __restrict__ logits,
    float* __restrict__ zero_ptr, size_t zero_words) {
  if (zero_ptr != nullptr && blockIdx.x == 0 && blockIdx.y == 0)
    for (size_t i = threadIdx.x; i < zero_words; i += 256) zero_ptr[i] = 0.0f;
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;   // whole wave; no barrier follows
  const int t0 = blockIdx.y * kGemvTokens;
  const int nchunk = H / 8;
  const u32x4* wrow = reinterpret_cast<const u32x4*>(wr + (size_t)e * H);
  const u32x4* xrow[kGemvTokens];
#pragma unroll
  for (int u = 0; u < kGemvTokens; ++u)
    xrow[u] = reinterpret_cast<const u32x4*>(x + (size_t)(t0 + u < M ? t0 + u : 0) * H);
  float acc[kGemvTokens];
#pragma unroll
  for (int u = 0; u < kGemvTokens; ++u) acc[u] = 0.f;
  for (int base = lane; base < nchunk + lane; base += 64 * NC) {
    u32x4 wv[NC], xv[kGemvTokens][NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = base + 64 * c;
      wv[c] = load16_or_zero(wrow + (ch < nchunk ? ch : 0), ch < nchunk);
#pragma unroll
      for (int u = 0; u < kGemvTokens; ++u)
        xv[u][c] = load16_or_zero(xrow[u] + (ch < nchunk ? ch : 0), ch < nchunk);
    }
#pragma unroll
    for (int u = 0; u < kGemvTokens; ++u)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[u] = __builtin_fmaf(__uint_as_float(wv[c][q] << 16),
                                  __uint_as_float(xv[u][c][q] << 16), acc[u]);
          acc[u] = __builtin_fmaf(__uint_as_float(wv[c][q] & 0xffff0000u),
                                  __uint_as_float(xv[u][c][q] & 0xffff0000u), acc[u]);
        }
  }
  const float b = bias != nullptr ? bias[e] : 0.f;
#pragma unroll
  for (int u = 0; u < kGemvTokens; ++u) {
    const float v = wave_sum(acc[u]);
    if (lane == 0 && t0 + u < M) logits[(size_t)(t0 + u) * E + e] = v + b;
  }
}

// Router logits for large batches: LDS-tiled MFMA GEMM over a tile of BT
// tokens (32 or 64) x EX experts (32, 64 or 128), 4 waves (2 expert halves
// x 2 token halves, each EX/2 experts x BT/2 tokens).  K goes through LDS in stages of
// KS sub-tiles of 64 elements, three stages deep, copied with
// global_load_lds_dwordx4; a sub-tile's rows are 128 bytes with chunk c of
// row R at slot c ^ ((R >> 1) & 7) (conflict-free operand reads).  Expert
// rows and token rows past the ends, and the K tail, copy a zeroed page.
// Each W_r tile is read by M/BT workgroups and each token row by E/EX, all
// other reuse comes from LDS; the host picks the tile that moves the fewest
// bytes per CU.  The grid is about one workgroup per CU, so a stage holds as
// many sub-tiles as 144 KB of LDS allows: fewer, larger stages keep more
// bytes in flight per CU than 64-element stages.
constexpr int kRtBK = 64;
constexpr int kRtStages = 3;
constexpr int kRtMaxLds = 144 * 1024;
template <int BT, int EX>
struct RtCfg {
  static constexpr int kRows = EX + BT;
  static constexpr int KS = 3 * 4 * kRows * 128 <= kRtMaxLds ? 4 : 3 * 2 * kRows * 128 <= kRtMaxLds ? 2 : 1;
  static constexpr int kLds = kRtStages * KS * kRows * 128;
};

__device__ __forceinline__ int rt_swz(int row) { return (row >> 1) & 7; }

template <int BT, int EX>
__global__ __launch_bounds__(256) void route_logits_tiled_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int M, int H, int E, float* __restrict__ logits,
    float* __restrict__ zero_ptr, size_t zero_words) {
  constexpr int kRows = EX + BT;
  constexpr int KS = RtCfg<BT, EX>::KS;      // 64-element sub-tiles per stage
  constexpr int kSubBytes = kRows * 128;
  constexpr int kStageBytes = KS * kSubBytes;
  constexpr int kCopies = kRows / 8 / 4;     // 1 KB copies per wave per sub-tile
  constexpr int NTA = EX / 32;               // 16-expert MFMA tiles per wave
  constexpr int NTB = BT / 32;               // 16-token MFMA tiles per wave
  static_assert(kCopies * 32 == kRows, "copies cover the stage");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  if (zero_ptr != nullptr && blockIdx.x == 0 && blockIdx.y == 0)
    for (size_t i = threadIdx.x; i < zero_words; i += 256) zero_ptr[i] = 0.0f;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lrow = lane >> 3, lpos = lane & 7;
  const int t0 = blockIdx.x * BT, e0 = blockIdx.y * EX;
  const uint16_t* zero = reinterpret_cast<const uint16_t*>(kZeroPage);
  // copy sources: rows 0..EX-1 experts, EX.. tokens
  const uint16_t* src[kCopies];
#pragma unroll
  for (int c = 0; c < kCopies; ++c) {
    const int R = (wv * kCopies + c) * 8 + lrow;
    const uint16_t* row = nullptr;
    if (R < EX) {
      if (e0 + R < E) row = wr + (size_t)(e0 + R) * H;
    } else if (t0 + R - EX < M) {
      row = x + (size_t)(t0 + R - EX) * H;
    }
    src[c] = row != nullptr ? row + (lpos ^ rt_swz(R)) * 8 : nullptr;
  }
  const int nk = ceil_div(H, kRtBK * KS);
  auto issue = [&](int kt) {
    uint8_t* sb = lds + (kt % kRtStages) * kStageBytes;
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const int k0 = (kt * KS + u) * kRtBK;
      const int kend = H - k0;   // valid elements of this sub-tile (may be <= 0)
#pragma unroll
      for (int c = 0; c < kCopies; ++c) {
        const int R = (wv * kCopies + c) * 8 + lrow;
        const uint16_t* p = (src[c] != nullptr && (lpos ^ rt_swz(R)) * 8 < kend)
                                ? src[c] + k0 : zero;
        load_lds16(p, sb + u * kSubBytes + (wv * kCopies + c) * 1024);
      }
    }
  };

  const int we = (wv & 1) * (EX / 2), wt = (wv >> 1) * (BT / 2);
  const int r16 = lane & 15, kg = lane >> 4;
  int abase[2], bbase[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int slot = ((s * 4 + kg) ^ rt_swz(r16)) << 4;
    abase[s] = (we + r16) * 128 + slot;
    bbase[s] = (EX + wt + r16) * 128 + slot;
  }
  f32x4 acc[NTA][NTB];
#pragma unroll
  for (int i = 0; i < NTA; ++i)
#pragma unroll
    for (int j = 0; j < NTB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0);
  if (nk > 1) issue(1);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) wait_vmem<KS * kCopies>(); else wait_vmem<0>();
    barrier_nofence();
    if (kt + 2 < nk) issue(kt + 2);
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const uint8_t* sb = lds + (kt % kRtStages) * kStageBytes + u * kSubBytes;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 af[NTA], bfr[NTB];
#pragma unroll
        for (int i = 0; i < NTA; ++i) af[i] = *reinterpret_cast<const u32x4*>(sb + abase[s] + i * 16 * 128);
#pragma unroll
        for (int j = 0; j < NTB; ++j) bfr[j] = *reinterpret_cast<const u32x4*>(sb + bbase[s] + j * 16 * 128);
#pragma unroll
        for (int i = 0; i < NTA; ++i)
#pragma unroll
          for (int j = 0; j < NTB; ++j) acc[i][j] = mfma_16x16x32(af[i], bfr[j], acc[i][j]);
      }
    }
  }
  // C: lane holds experts e0 + we + 16 i + 4 kg + q for token t0 + wt + 16 j + r16.
#pragma unroll
  for (int j = 0; j < NTB; ++j) {
    const int t = t0 + wt + 16 * j + r16;
    if (t >= M) continue;
#pragma unroll
    for (int i = 0; i < NTA; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + we + 16 * i + 4 * kg + q;
        if (e < E) logits[(size_t)t * E + e] = acc[i][j][q] + (bias != nullptr ? bias[e] : 0.f);
      }
  }
}

// Softmax over all E, ordered top-k, renormalize; one wave per token.  With
// qx non-null the workgroup also writes the MXFP8 codes and scales of its
// four tokens' x rows (the quantized GEMM 1 input of the MXFP8 layer, page
// "Mixture of Experts in vLLM ...", sub-section "The two index lists":
// qhidden), so that no separate launch is needed.
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int M, int E, int top_k, int renormalize,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights,
    const uint16_t* __restrict__ x, int H, uint8_t* __restrict__ qx, uint8_t* __restrict__ qxs) {
  __shared__ __attribute__((aligned(16))) float scratch[4][topk_wave_floats(512)];
  if (qx != nullptr) {
    const long long nb = H / 32;
    const long long b0 = (long long)blockIdx.x * 4 * nb;
    const long long b1 = (long long)min(M, (int)blockIdx.x * 4 + 4) * nb;
    for (long long b = b0 + threadIdx.x; b < b1; b += 256) mx_quantize_block(x, H, b, qx, qxs);
  }
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  if (t >= M) return;   // whole wave; no workgroup barrier below
  const TopkSlot r = topk_token(logits + (size_t)t * E, E, top_k, renormalize, scratch[w]);
  if ((threadIdx.x & 63) < top_k) {
    topk_ids[(size_t)t * top_k + (threadIdx.x & 63)] = r.id;
    topk_weights[(size_t)t * top_k + (threadIdx.x & 63)] = r.w;
  }
}

}  // namespace

namespace moe_host {

// Small batches split K over the waves (more workgroups read W_r at once);
// larger ones use the LDS-tiled kernel.
constexpr int kSmallMaxTokens = 256;

// Batches up to this many tokens use the GEMV-style kernel.
constexpr int kGemvMaxTokens = 16;

template <int NC>
void launch_route_gemv(const RouteArgs& a, hipStream_t s) {
  dim3 grid(ceil_div_host(a.E, 4), ceil_div_host(a.M, kGemvTokens));
  hipLaunchKernelGGL(route_logits_gemv_kernel<NC>, grid, dim3(256), 0, s, a.x, a.w_router, a.bias,
                     a.M, a.H, a.E, a.logits, a.zero_ptr, a.zero_words);
}

hipError_t launch_route_logits(const RouteArgs& a, hipStream_t s) {
  if (a.M <= kGemvMaxTokens) {
    const int n = (a.H / 8 + 63) / 64;   // chunks per lane covering H, at most 4 per pass
    switch (n <= 1 ? 1 : (n >= 4 ? 4 : n)) {
      case 1: launch_route_gemv<1>(a, s); break;
      case 2: launch_route_gemv<2>(a, s); break;
      case 3: launch_route_gemv<3>(a, s); break;
      default: launch_route_gemv<4>(a, s); break;
    }
  } else if (a.M <= kSmallMaxTokens) {
    dim3 grid(ceil_div_host(a.M, kTokTile), ceil_div_host(a.E, 16));
    hipLaunchKernelGGL(route_logits_small_kernel, grid, dim3(256), 0, s, a.x, a.w_router,
                       a.bias, a.M, a.H, a.E, a.logits, a.zero_ptr, a.zero_words);
  } else {
    // the (tokens, experts) tile that moves the fewest bytes per CU: rounds
    // of workgroups over the CUs times each workgroup's rows
    const int cus = device_cu_count();
    int best_bt = 64, best_ex = 128;
    long long best = -1;
    for (int bt : {32, 64})
      for (int ex : {32, 64, 128}) {
        const long long wgs = (long long)ceil_div_host(a.M, bt) * ceil_div_host(a.E, ex);
        const long long cost = (wgs + cus - 1) / cus * (bt + ex);
        if (best < 0 || cost < best) { best = cost; best_bt = bt; best_ex = ex; }
      }
    dim3 grid(ceil_div_host(a.M, best_bt), ceil_div_host(a.E, best_ex));
    hipError_t e = hipSuccess;
    auto go = [&](auto kern, int lds, bool (&lds_set)[kMaxDevices]) {
      // stages above the default limit of dynamic LDS
      e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), lds, lds_set);
      if (e != hipSuccess) return;
      hipLaunchKernelGGL(kern, grid, dim3(256), (size_t)lds, s, a.x, a.w_router, a.bias, a.M, a.H,
                         a.E, a.logits, a.zero_ptr, a.zero_words);
    };
    static bool set[6][kMaxDevices] = {};
    switch (best_bt * 1000 + best_ex) {
      case 32032: go(route_logits_tiled_kernel<32, 32>, RtCfg<32, 32>::kLds, set[0]); break;
      case 32064: go(route_logits_tiled_kernel<32, 64>, RtCfg<32, 64>::kLds, set[1]); break;
      case 32128: go(route_logits_tiled_kernel<32, 128>, RtCfg<32, 128>::kLds, set[2]); break;
      case 64032: go(route_logits_tiled_kernel<64, 32>, RtCfg<64, 32>::kLds, set[3]); break;
      case 64064: go(route_logits_tiled_kernel<64, 64>, RtCfg<64, 64>::kLds, set[4]); break;
      default: go(route_logits_tiled_kernel<64, 128>, RtCfg<64, 128>::kLds, set[5]); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_route_topk(const RouteArgs& a, hipStream_t s) {
  dim3 grid(ceil_div_host(a.M, 4));
  hipLaunchKernelGGL(route_topk_kernel, grid, dim3(256), 0, s, a.logits, a.M, a.E, a.top_k,
                     a.renormalize, a.topk_ids, a.topk_weights, a.x, a.H, a.qx_codes,
                     a.qx_scales);
  return hipGetLastError();
}

}  // namespace moe_host
