// Weight-streaming grouped GEMMs for small batches (about one pair per
// expert).  Page "Mixture of Experts in vLLM - From First Principles to
// fused_moe", sub-section "Each expert is now an ordinary GEMM": with n_e
// near 1 each expert reads all of its weights to make about one output row,
// so the cost is the weight bytes and the kernel's job is to stream them at
// full HBM bandwidth.
//
// Blocks of 16 pairs (index lists built with block_m = 16).  Weight rows
// stream directly from HBM into registers with 16-byte loads in the MFMA
// operand layout: lane l owns row (l % 16) of a 16-row tile, and for the
// s-th 32-element k step of a 256-element super-chunk it loads elements
// 32 s + 8 g .. + 7 (g = l / 16), so the four lanes of a row read 64
// contiguous bytes per load instruction and consecutive instructions walk
// along the row.  The gathered pair rows are loaded the same way as the B
// operand, so one 16x16x32 MFMA per load does the dot products with no
// cross-lane reduction.  Pads (id >= M*top_k) load zeros and store nothing.
//
// GEMM 1: a workgroup owns 16 gate rows and the matching 16 up rows of
//   W13[e]; its 4 waves split K (super-chunks w, w+4, ...) and add their
//   partial tiles through LDS; wave 0 applies SiLU(gate) * up and writes
//   act rows p (pair order).
// GEMM 2: a workgroup owns 64 rows of W2[e] (16 per wave, full K); the
//   epilogue scales by topk_weights[p] and stores fp32 partial row p; the
//   last of the top_k workgroups producing a (token, 64 columns) piece adds
//   the token's partial rows in slot order and writes it as bf16 (page
//   sections "Put the results back, and combine them per token" and "The
//   rest of the layer stays in pair order").
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kBM = 16;
constexpr int kSC = 256;   // k elements per super-chunk (8 MFMA k steps of 32)

__global__ __launch_bounds__(256) void gemm1_stream_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w13,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ expert_ids,
    const int32_t* __restrict__ boff, int M, int top_k, int E, int H, int I,
    uint16_t* __restrict__ act) {
  __shared__ f32x4 red[4][2][64];
  const int b = blockIdx.x;
  if (b >= boff[E]) return;
  const int P = M * top_k;
  const int e = expert_ids[b];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n = blockIdx.y * 16 + r;
  const bool n_ok = n < I;
  const uint16_t* gp = w13 + ((size_t)e * 2 * I + (n_ok ? n : 0)) * H;
  const uint16_t* up = gp + (size_t)I * H;
  const int p = sorted[b * kBM + r];
  const bool p_ok = p < P;
  const uint16_t* xp = x + (size_t)(p_ok ? p / top_k : 0) * H;

  f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  const int nsc = ceil_div(H, kSC);
  for (int sc = wv; sc < nsc; sc += 4) {
    const int kb = sc * kSC + g * 8;
    u32x4 ga[8], ua[8], xb[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int k = kb + s * 32;
      const bool kin = k < H;
      ga[s] = load16_or_zero(gp + k, n_ok && kin);
      ua[s] = load16_or_zero(up + k, n_ok && kin);
      xb[s] = load16_or_zero(xp + k, p_ok && kin);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      accg = mfma_16x16x32(ga[s], xb[s], accg);
      accu = mfma_16x16x32(ua[s], xb[s], accu);
    }
  }
  red[wv][0][lane] = accg;
  red[wv][1][lane] = accu;
  __syncthreads();
  if (wv != 0) return;
  f32x4 gs = red[0][0][lane], us = red[0][1][lane];
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    gs += red[i][0][lane];
    us += red[i][1][lane];
  }
  // lane holds features blockIdx.y*16 + 4g + q of pair column r
  const int nf = blockIdx.y * 16 + 4 * g;
  if (p_ok && nf < I) {
    u32x2 v;
    v[0] = pack_bf16x2(silu_mul(gs[0], us[0]), silu_mul(gs[1], us[1]));
    v[1] = pack_bf16x2(silu_mul(gs[2], us[2]), silu_mul(gs[3], us[3]));
    *reinterpret_cast<u32x2*>(act + (size_t)p * I + nf) = v;
  }
}

__global__ __launch_bounds__(256) void gemm2_stream_kernel(
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

}  // namespace

namespace moe_host {

hipError_t launch_gemm1_stream(const GemmArgs& a, hipStream_t s) {
  dim3 grid(a.max_blocks, ceil_div_host(a.I, 16));
  hipLaunchKernelGGL(gemm1_stream_kernel, grid, dim3(256), 0, s, a.a_src, a.w,
                     a.sorted_token_ids, a.expert_ids, a.expert_block_offsets, a.M, a.top_k,
                     a.E, a.H, a.I, a.out);
  return hipGetLastError();
}

hipError_t launch_gemm2_stream(const GemmArgs& a, hipStream_t s) {
  dim3 grid(a.max_blocks, ceil_div_host(a.H, 64));
  hipLaunchKernelGGL(gemm2_stream_kernel, grid, dim3(256), 0, s, a.a_src, a.w, a.topk_weights,
                     a.sorted_token_ids, a.expert_ids, a.expert_block_offsets, a.M, a.top_k,
                     a.E, a.H, a.I, a.out, a.partial, a.counters);
  return hipGetLastError();
}

}  // namespace moe_host
