// Per-pair GEMVs for very small batches (M*top_k*4 <= E).
//
// Page "Mixture of Experts in vLLM - From First Principles to fused_moe",
// sub-section "Small batches skip the sort": with this few pairs there is no
// grouping to exploit; each pair (token t, slot j) is a one-row product
// against its own expert's weights, which it reads once.  The cost is the
// weight bytes, so the kernels keep many 16-byte loads per lane in flight:
// a wave reads whole weight rows (lane l takes the 16-byte chunks l, l + 64,
// ... of a row), multiplies them by the token's row held in registers in the
// same chunk order, and a wave reduction gives each dot product.  The expert
// of pair p is read straight from topk_ids[p]: no index lists, no MFMA.
//
// GEMM 1 (sub-section "One GEMM 1 program, step by step", one pair per
//   program): a workgroup owns one pair and 16 act columns, wave w the four
//   features f0 = 16*blockIdx.x + 4w .. f0 + 3, i.e. four gate rows and the
//   matching four up rows of W13[e];
//   act[p, f] = SiLU(gate_f . x_t) * (up_f . x_t), fp32, stored once as bf16.
// GEMM 2 with the combine (sections "The rest of the layer stays in pair
//   order" and "Put the results back, and combine them per token"): a
//   workgroup owns one token and 8 output columns, wave w the slots
//   j = w, w + nwaves, ...; for each column h it accumulates
//   topk_weights[t, j] * (W2[e_j][h] . act[t*top_k + j]) over its slots, and
//   the waves' sums are added in wave order (a fixed order: bitwise
//   repeatable), then rounded once to bf16.
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kW13Threads = 256;       // 4 waves x 4 features
constexpr int kW13Features = 16;       // act columns per GEMM 1 workgroup
constexpr int kW2Rows = 8;             // output columns per GEMM 2 workgroup
constexpr int kW2MaxWaves = 8;

// Sum over this lane's NC chunks of 8 bf16 products, in fp32.
template <int NC>
__device__ __forceinline__ float dot_chunks(const u32x4 (&a)[NC], const u32x4 (&b)[NC], float s) {
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s = __builtin_fmaf(__uint_as_float(a[c][q] << 16), __uint_as_float(b[c][q] << 16), s);
      s = __builtin_fmaf(__uint_as_float(a[c][q] & 0xffff0000u),
                         __uint_as_float(b[c][q] & 0xffff0000u), s);
    }
  return s;
}

// Chunk `chunk` (16 bytes) of a row of nchunk chunks, zeros past its end.
// The load is issued for every lane (from the row start when past the end)
// so that all loads of a pass leave back to back without branches.
template <bool kStream>
__device__ __forceinline__ u32x4 chunk_or_zero(const uint16_t* row, int chunk, int nchunk) {
  const bool ok = chunk < nchunk;
  const u32x4* p = reinterpret_cast<const u32x4*>(row + (size_t)(ok ? chunk : 0) * 8);
  u32x4 v = kStream ? __builtin_nontemporal_load(p) : *p;
  if (!ok) v = u32x4{0u, 0u, 0u, 0u};
  return v;
}

// NC = 16-byte chunks per lane per pass: one pass covers 512*NC elements of K.
template <int NC>
__global__ __launch_bounds__(kW13Threads) void gemv_w13_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w13,
    const int32_t* __restrict__ topk_ids, int top_k, int H, int I, uint16_t* __restrict__ act) {
  const int p = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int f0 = blockIdx.x * kW13Features + (threadIdx.x >> 6) * 4;
  // I % 8 == 0 and f0 % 4 == 0: a wave's four features are all valid or all past I
  if (f0 >= I) return;
  const int t = p / top_k;
  const int e = topk_ids[p];
  const int nchunk = H / 8;
  const uint16_t* xrow = x + (size_t)t * H;
  const uint16_t* gate = w13 + ((size_t)e * 2 * I + f0) * H;   // rows f0..f0+3
  const uint16_t* up = gate + (size_t)I * H;                   // rows I+f0..
  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.f;
  for (int base = lane; base < nchunk + lane; base += 64 * NC) {
    u32x4 wv[8][NC];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        wv[r][c] = chunk_or_zero<true>((r < 4 ? gate : up) + (size_t)(r & 3) * H, base + 64 * c,
                                       nchunk);
    u32x4 xv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) xv[c] = chunk_or_zero<false>(xrow, base + 64 * c, nchunk);
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = dot_chunks<NC>(wv[r], xv, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
    u32x2 v;
    v[0] = pack_bf16x2(silu_mul(acc[0], acc[4]), silu_mul(acc[1], acc[5]));
    v[1] = pack_bf16x2(silu_mul(acc[2], acc[6]), silu_mul(acc[3], acc[7]));
    *reinterpret_cast<u32x2*>(act + (size_t)p * I + f0) = v;
  }
}

template <int NC>
__global__ __launch_bounds__(64 * kW2MaxWaves) void gemv_w2_sum_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_weights, int top_k,
    int H, int I, uint16_t* __restrict__ out) {
  __shared__ float red[kW2MaxWaves][kW2Rows];
  const int t = blockIdx.y;
  const int h0 = blockIdx.x * kW2Rows;   // H % 8 == 0: all 8 rows exist
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int nchunk = I / 8;
  float acc[kW2Rows];
#pragma unroll
  for (int r = 0; r < kW2Rows; ++r) acc[r] = 0.f;
  for (int j = w; j < top_k; j += nwaves) {
    const int p = t * top_k + j;
    const int e = topk_ids[p];
    const float wt = topk_weights[p];
    const uint16_t* arow = act + (size_t)p * I;
    const uint16_t* wrow = w2 + ((size_t)e * H + h0) * I;
    float s[kW2Rows];
#pragma unroll
    for (int r = 0; r < kW2Rows; ++r) s[r] = 0.f;
    for (int base = lane; base < nchunk + lane; base += 64 * NC) {
      u32x4 wv[kW2Rows][NC];
#pragma unroll
      for (int r = 0; r < kW2Rows; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          wv[r][c] = chunk_or_zero<true>(wrow + (size_t)r * I, base + 64 * c, nchunk);
      u32x4 av[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) av[c] = chunk_or_zero<false>(arow, base + 64 * c, nchunk);
#pragma unroll
      for (int r = 0; r < kW2Rows; ++r) s[r] = dot_chunks<NC>(wv[r], av, s[r]);
    }
#pragma unroll
    for (int r = 0; r < kW2Rows; ++r) acc[r] = __builtin_fmaf(wt, s[r], acc[r]);
  }
#pragma unroll
  for (int r = 0; r < kW2Rows; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == 0) red[w][r] = v;
  }
  __syncthreads();
  if (threadIdx.x < kW2Rows) {
    float v = red[0][threadIdx.x];
    for (int i = 1; i < nwaves; ++i) v += red[i][threadIdx.x];
    out[(size_t)t * H + h0 + threadIdx.x] = (uint16_t)f32_to_bf16(v);
  }
}

// Chunks per lane per pass for a K of k elements: enough to cover K in one
// pass up to 2048, then passes of 2048.
int chunks_per_lane(int k) {
  const int n = (k / 8 + 63) / 64;
  return n < 1 ? 1 : (n > 4 ? 4 : n);
}

template <int NC>
void launch_w13(const moe_host::PairGemvArgs& a, hipStream_t s) {
  dim3 grid(moe_host::ceil_div_host(a.I, kW13Features), a.M * a.top_k);
  hipLaunchKernelGGL(gemv_w13_kernel<NC>, grid, dim3(kW13Threads), 0, s, a.x, a.w13, a.topk_ids,
                     a.top_k, a.H, a.I, a.act);
}

template <int NC>
void launch_w2(const moe_host::PairGemvArgs& a, hipStream_t s) {
  const int waves = a.top_k < kW2MaxWaves ? a.top_k : kW2MaxWaves;
  dim3 grid(a.H / kW2Rows, a.M);
  hipLaunchKernelGGL(gemv_w2_sum_kernel<NC>, grid, dim3(64 * waves), 0, s, a.act, a.w2,
                     a.topk_ids, a.topk_weights, a.top_k, a.H, a.I, a.out);
}

}  // namespace

namespace moe_host {

hipError_t launch_pair_gemv1(const PairGemvArgs& a, hipStream_t s) {
  switch (chunks_per_lane(a.H)) {
    case 1: launch_w13<1>(a, s); break;
    case 2: launch_w13<2>(a, s); break;
    case 3: launch_w13<3>(a, s); break;
    default: launch_w13<4>(a, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_pair_gemv2(const PairGemvArgs& a, hipStream_t s) {
  switch (chunks_per_lane(a.I)) {
    case 1: launch_w2<1>(a, s); break;
    case 2: launch_w2<2>(a, s); break;
    case 3: launch_w2<3>(a, s); break;
    default: launch_w2<4>(a, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe_host
