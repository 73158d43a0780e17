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
// kSplitK = true  (small batches): a workgroup owns 16 tokens x 16 experts
//   and its 4 waves split K in four contiguous ranges; partial tiles are
//   added through LDS.  Many workgroups read W_r in parallel.
// kSplitK = false (large batches): a workgroup owns 16 tokens x 64 experts,
//   wave w the 16 experts 16 w .. 16 w + 15 over the whole K.
// grid: (ceil(M / 16), ceil(E / experts per workgroup)); block: 256.
template <bool kSplitK>
__global__ __launch_bounds__(256) void route_logits_kernel(
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
  const int e0 = kSplitK ? blockIdx.y * 16 : blockIdx.y * 64 + w * 16;
  const int erow = e0 + r, trow = t0 + r;
  const bool e_ok = erow < E, t_ok = trow < M;
  const uint16_t* ap = wr + (size_t)(e_ok ? erow : 0) * H;
  const uint16_t* bp = x + (size_t)(t_ok ? trow : 0) * H;
  int kbeg = 0, kend = H;
  if (kSplitK) {
    const int kw = ceil_div(ceil_div(H, 4), 32) * 32;
    kbeg = min(H, w * kw);
    kend = min(H, kbeg + kw);
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (!kSplitK && e0 >= E) {
    // no experts for this wave
  } else {
    constexpr int U = kSplitK ? 16 : 8;   // k steps whose loads are in flight together
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
  }
  if (kSplitK) {
    red[w][lane] = acc;
    __syncthreads();
    if (w != 0) return;
    acc = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
  }
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

// Softmax over all E, ordered top-k, renormalize; one wave per token.
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int M, int E, int top_k, int renormalize,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights) {
  __shared__ __attribute__((aligned(16))) float scratch[4][topk_wave_floats(512)];
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

// Small batches split K over the waves (more workgroups read W_r at once).
constexpr int kSplitKMaxTokens = 256;

hipError_t launch_route_logits(const RouteArgs& a, hipStream_t s) {
  if (a.M <= kSplitKMaxTokens) {
    dim3 grid(ceil_div_host(a.M, kTokTile), ceil_div_host(a.E, 16));
    hipLaunchKernelGGL(route_logits_kernel<true>, grid, dim3(256), 0, s, a.x, a.w_router,
                       a.bias, a.M, a.H, a.E, a.logits, a.zero_ptr, a.zero_words);
  } else {
    dim3 grid(ceil_div_host(a.M, kTokTile), ceil_div_host(a.E, 64));
    hipLaunchKernelGGL(route_logits_kernel<false>, grid, dim3(256), 0, s, a.x, a.w_router,
                       a.bias, a.M, a.H, a.E, a.logits, a.zero_ptr, a.zero_words);
  }
  return hipGetLastError();
}

hipError_t launch_route_topk(const RouteArgs& a, hipStream_t s) {
  dim3 grid(ceil_div_host(a.M, 4));
  hipLaunchKernelGGL(route_topk_kernel, grid, dim3(256), 0, s, a.logits, a.M, a.E, a.top_k,
                     a.renormalize, a.topk_ids, a.topk_weights);
  return hipGetLastError();
}

}  // namespace moe_host
