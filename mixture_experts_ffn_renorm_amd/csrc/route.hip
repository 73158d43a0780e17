// Router: logits = W_r x (MFMA, fp32 accumulate), then per token softmax
// over all experts, ordered top-k (exact ties -> lower id) and renormalize.
// Page "Mixture of Experts in vLLM - From First Principles to fused_moe",
// section "One expert, and one token", sub-section "One token uses only 8
// experts".
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kTokTile = 16;     // tokens per workgroup (MFMA B columns)
constexpr int kExpTile = 64;     // experts per workgroup (4 waves x 16 rows)
constexpr int kKChunk = 128;     // k elements per lane-group sweep (4 MFMAs)

// grid: (ceil(M/16), ceil(E/64)); block: 256 threads.
// Wave w computes logits of experts e0 = by*64 + 16w .. +15 for the 16 tokens
// of the tile.  Lane l: row/col r = l % 16, k group g = l / 16.  Within a
// 128-element k chunk the lane loads the 32 contiguous elements
// [g*32, g*32+32) of its W_r row and of its token row; MFMA s (0..3) pairs
// elements g*32 + 8s .. +7 of both, so each chunk is summed exactly once.
__global__ __launch_bounds__(256) void route_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int M, int H, int E, float* __restrict__ logits,
    float* __restrict__ zero_ptr, size_t zero_words) {
  // Optional clearing of the combine scratch (fp32 sums + counters) for the
  // GEMM 2 that follows on the same stream.
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

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * kTokTile;
  const int e0 = blockIdx.y * kExpTile + w * 16;
  if (e0 >= E) return;
  const int erow = e0 + r, trow = t0 + r;
  const bool e_ok = erow < E, t_ok = trow < M;
  const uint16_t* ap = wr + (size_t)(e_ok ? erow : 0) * H;
  const uint16_t* bp = x + (size_t)(t_ok ? trow : 0) * H;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < H; kc += kKChunk) {
    u32x4 av[4], bv[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = kc + g * 32 + s * 8;
      const bool kin = k < H;  // H % 8 == 0, so k < H means all 8 fit
      av[s] = load16_or_zero(ap + k, e_ok && kin);
      bv[s] = load16_or_zero(bp + k, t_ok && kin);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_16x16x32(av[s], bv[s], acc);
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

// One wave per token.  Lane l owns experts l, l+64, ... (E <= 512).
// Softmax over all E (fp32, max-shifted), then k rounds of a wave argmax on
// (logit desc, expert id asc); the probability of the winner is
// exp(l - max) / sum.  Renormalize divides by the sum of the k kept values.
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int M, int E, int top_k, int renormalize,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= M) return;
  constexpr int kMaxPerLane = 8;
  float v[kMaxPerLane];
  const float* row = logits + (size_t)t * E;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
  }
  float m = v[0];
#pragma unroll
  for (int i = 1; i < kMaxPerLane; ++i) m = fmaxf(m, v[i]);
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i)
    if (lane + 64 * i < E) s += __expf(v[i] - m);
  s = wave_sum(s);

  uint32_t taken = 0;
  int my_id = 0;
  float my_p = 0.f;
  for (int j = 0; j < top_k; ++j) {
    // best untaken candidate of this lane (ids increase with i, so strict >
    // keeps the lower id on ties)
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || bi == 0x7FFFFFFF)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d, kWave);
      const int oi = __shfl_xor(bi, d, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      my_id = bi;
      my_p = __expf(bv - m) / s;
    }
  }
  float tot = wave_sum(lane < top_k ? my_p : 0.f);
  if (lane < top_k) {
    topk_ids[(size_t)t * top_k + lane] = my_id;
    topk_weights[(size_t)t * top_k + lane] = renormalize ? my_p / tot : my_p;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, size_t words) {
  const size_t n4 = words >> 2;
  const size_t stride = (size_t)gridDim.x * 256;
  u32x4 z = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride)
    reinterpret_cast<u32x4*>(p)[i] = z;
  for (size_t i = (n4 << 2) + (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += stride)
    p[i] = 0.0f;
}

}  // namespace

namespace moe_host {

hipError_t launch_route_logits(const RouteArgs& a, hipStream_t s) {
  dim3 grid(ceil_div_host(a.M, kTokTile), ceil_div_host(a.E, kExpTile));
  hipLaunchKernelGGL(route_logits_kernel, grid, dim3(256), 0, s, a.x, a.w_router, a.bias, a.M,
                     a.H, a.E, a.logits, a.zero_ptr, a.zero_words);
  return hipGetLastError();
}

hipError_t launch_route_topk(const RouteArgs& a, hipStream_t s) {
  dim3 grid(ceil_div_host(a.M, 4));
  hipLaunchKernelGGL(route_topk_kernel, grid, dim3(256), 0, s, a.logits, a.M, a.E, a.top_k,
                     a.renormalize, a.topk_ids, a.topk_weights);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t words, hipStream_t s) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words / 4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, words);
  return hipGetLastError();
}

}  // namespace moe_host
