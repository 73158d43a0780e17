// Per-pair GEMVs for very small batches (M*top_k*4 <= E).
//
// Page "Mixture of Experts in vLLM - From First Principles to fused_moe",
// sub-section "Small batches skip the sort": with this few pairs there is no
// grouping to exploit; each pair (token t, slot j) is a one-row product
// against its own expert's weights, which it reads once, and the expert of
// pair p is read straight from topk_ids[p] (no index lists, no MFMA).  The
// cost is the weight bytes and the latency of each step, so the kernels run
// many small workgroups that all fit on the chip at once; each issues all of
// its 16-byte loads before it waits: a wave reads whole weight rows (lane l
// takes the 16-byte chunks l, l + 64, ... of a row), multiplies them by the
// token's row held in registers in the same chunk order, and a wave
// reduction gives each dot product.
//
// The per-step GEMM calls reach the same kernels with block_m 1: index lists
// of one pair per block (no pads), block b holding pair sorted[b] of expert
// expert_ids[b]; GEMV 1 is the same kernel in that order, and GEMV 2 then
// writes fp32 rows of pair p, already scaled by topk_weights[p], for the
// per-token sum kernel (it has no topk_ids to group a token's pairs).
//
// GEMV 1 (sub-section "One GEMM 1 program, step by step", one pair per
//   program): a workgroup owns one pair p and 4*FW act columns, wave w the FW
//   columns f0 = (4 blockIdx.x + w) FW ..: gate rows f of W13[e] and the
//   matching up rows I + f;
//   act[p, f] = SiLU(gate_f . x_t) * (up_f . x_t), fp32, rounded once to bf16.
// GEMV 2 with the combine (sections "The rest of the layer stays in pair
//   order" and "Put the results back, and combine them per token"): a
//   workgroup owns token t and R output columns h0 .. h0 + R - 1, wave w its
//   slots j = w, w + nwaves, ...; a wave adds
//   topk_weights[t, j] * (W2[e_j][h] . act[t*top_k + j]) over its slots; the
//   waves' sums are added in wave order (a fixed order: bitwise repeatable)
//   and rounded once to bf16.
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kG1Waves = 4;    // GEMV 1: waves per workgroup
constexpr int kG1Cols = 1;     // GEMV 1: act columns per wave (divides 8)
constexpr int kMaxWaves = 8;   // GEMV 2: waves per workgroup, min(top_k, 8)
constexpr int kG2Cols = 4;     // GEMV 2: output columns per workgroup (divides 8)

// Sum over this lane's NC chunks of 8 bf16 products, in fp32: the bf16
// dot-2 instruction takes two adjacent elements of each operand as they sit
// in memory (products exact in fp32, accumulated in fp32), so nothing is
// unpacked.

// (the words come in by value: a bit cast of a vector-element lvalue would
// read the vector's first element)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

template <int NC>
__device__ __forceinline__ float dot_chunks(const u32x4 (&a)[NC], const u32x4 (&b)[NC], float s) {
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) s = dot2_bf16(a[c][q], b[c][q], s);
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
// Block b = blockIdx.y: pair p = b and expert ids[p] (ids = topk_ids), or,
// with index lists, pair sorted[b] and expert ids[b] (ids = expert_ids).
template <int NC, int FW>
__global__ __launch_bounds__(64 * kG1Waves) void gemv_w13_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w13,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ ids, int top_k, int H, int I,
    uint16_t* __restrict__ act) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int f0 = (blockIdx.x * kG1Waves + (threadIdx.x >> 6)) * FW;
  // I % 8 == 0 and FW divides 8: a wave's columns are all valid or all past I
  if (f0 >= I) return;   // whole wave; no barrier follows
  const int p = sorted != nullptr ? sorted[b] : b;
  const int e = ids[b];
  const int nchunk = H / 8;
  const uint16_t* xrow = x + (size_t)(p / top_k) * H;
  const uint16_t* gate = w13 + ((size_t)e * 2 * I + f0) * H;   // rows f0 ..
  const uint16_t* up = gate + (size_t)I * H;                   // rows I + f0 ..
  float acc[2 * FW];
#pragma unroll
  for (int r = 0; r < 2 * FW; ++r) acc[r] = 0.f;
  for (int base = lane; base < nchunk + lane; base += 64 * NC) {
    u32x4 xv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) xv[c] = chunk_or_zero<false>(xrow, base + 64 * c, nchunk);
    u32x4 wv[2 * FW][NC];
#pragma unroll
    for (int r = 0; r < 2 * FW; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        wv[r][c] = chunk_or_zero<true>((r < FW ? gate : up) + (size_t)(r % FW) * H,
                                       base + 64 * c, nchunk);
#pragma unroll
    for (int r = 0; r < 2 * FW; ++r) acc[r] = dot_chunks<NC>(wv[r], xv, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < 2 * FW; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
    uint16_t* dst = act + (size_t)p * I + f0;
#pragma unroll
    for (int r = 0; r < FW; ++r) dst[r] = (uint16_t)f32_to_bf16(silu_mul(acc[r], acc[FW + r]));
  }
}

template <int NC, int R>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_w2_sum_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_weights, int top_k,
    int H, int I, uint16_t* __restrict__ out) {
  __shared__ float red[kMaxWaves][R];
  const int t = blockIdx.y;
  const int h0 = blockIdx.x * R;   // H % 8 == 0 and R divides 8: all R rows exist
  const int lane = threadIdx.x & 63;
  // wave-uniform: the slot's expert id and weight come in through scalar loads
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;   // <= top_k
  const int nchunk = I / 8;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  for (int j = w; j < top_k; j += nwaves) {
    const int p = t * top_k + j;
    const float wt = topk_weights[p];
    const uint16_t* arow = act + (size_t)p * I;
    const uint16_t* wrow = w2 + ((size_t)topk_ids[p] * H + h0) * I;
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = 0.f;
    for (int base = lane; base < nchunk + lane; base += 64 * NC) {
      u32x4 av[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) av[c] = chunk_or_zero<false>(arow, base + 64 * c, nchunk);
      u32x4 wv[R][NC];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          wv[r][c] = chunk_or_zero<true>(wrow + (size_t)r * I, base + 64 * c, nchunk);
#pragma unroll
      for (int r = 0; r < R; ++r) s[r] = dot_chunks<NC>(wv[r], av, s[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf(wt, s[r], acc[r]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == 0) red[w][r] = v;
  }
  __syncthreads();
  if (threadIdx.x < R) {
    float v = red[0][threadIdx.x];
    for (int i = 1; i < nwaves; ++i) v += red[i][threadIdx.x];
    out[(size_t)t * H + h0 + threadIdx.x] = (uint16_t)f32_to_bf16(v);
  }
}

// GEMV 2, index-list form: block b = blockIdx.y holds pair p = sorted[b] of
// expert expert_ids[b]; wave w of the workgroup owns output columns
// h0 = 8 blockIdx.x + 2w and h0 + 1 and writes
// partial[p, h] = topk_weights[p] * (W2[e][h] . act[p]) in fp32.
template <int NC>
__global__ __launch_bounds__(256) void gemv_w2_rows_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ expert_ids,
    const float* __restrict__ topk_weights, int H, int I, float* __restrict__ partial) {
  constexpr int R = 2;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int h0 = blockIdx.x * 8 + (threadIdx.x >> 6) * R;   // H % 8 == 0: all rows exist
  const int p = sorted[b];
  const int e = expert_ids[b];
  const int nchunk = I / 8;
  const uint16_t* arow = act + (size_t)p * I;
  const uint16_t* wrow = w2 + ((size_t)e * H + h0) * I;
  float s[R];
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = 0.f;
  for (int base = lane; base < nchunk + lane; base += 64 * NC) {
    u32x4 av[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) av[c] = chunk_or_zero<false>(arow, base + 64 * c, nchunk);
    u32x4 wv[R][NC];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        wv[r][c] = chunk_or_zero<true>(wrow + (size_t)r * I, base + 64 * c, nchunk);
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = dot_chunks<NC>(wv[r], av, s[r]);
  }
  const float wt = topk_weights[p];
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = wave_sum(s[r]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) partial[(size_t)p * H + h0 + r] = wt * s[r];
  }
}

// Chunks per lane per pass for a K of k elements: enough to cover K in one
// pass up to 2048, then passes of 2048.
int chunks_per_lane(int k) {
  const int n = (k / 8 + 63) / 64;
  return n < 1 ? 1 : (n > 4 ? 4 : n);
}

int waves_for(int top_k) { return top_k < kMaxWaves ? top_k : kMaxWaves; }

template <int NC>
void launch_w13(const moe_host::PairGemvArgs& a, hipStream_t s) {
  dim3 grid(moe_host::ceil_div_host(a.I, kG1Waves * kG1Cols), a.M * a.top_k);
  const int32_t* ids = a.sorted != nullptr ? a.expert_ids : a.topk_ids;
  hipLaunchKernelGGL((gemv_w13_kernel<NC, kG1Cols>), grid, dim3(64 * kG1Waves), 0, s, a.x, a.w13,
                     a.sorted, ids, a.top_k, a.H, a.I, a.act);
}

template <int NC>
void launch_w2_rows(const moe_host::PairGemvArgs& a, hipStream_t s) {
  dim3 grid(a.H / 8, a.M * a.top_k);
  hipLaunchKernelGGL(gemv_w2_rows_kernel<NC>, grid, dim3(256), 0, s, a.act, a.w2, a.sorted,
                     a.expert_ids, a.topk_weights, a.H, a.I, a.partial);
}

template <int NC>
void launch_w2(const moe_host::PairGemvArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gemv_w2_sum_kernel<NC, kG2Cols>), dim3(a.H / kG2Cols, a.M),
                     dim3(64 * waves_for(a.top_k)), 0, s, a.act, a.w2, a.topk_ids, a.topk_weights,
                     a.top_k, a.H, a.I, a.out);
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
  if (a.sorted != nullptr) {
    switch (chunks_per_lane(a.I)) {
      case 1: launch_w2_rows<1>(a, s); break;
      case 2: launch_w2_rows<2>(a, s); break;
      case 3: launch_w2_rows<3>(a, s); break;
      default: launch_w2_rows<4>(a, s); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_combine_partials(a.partial, a.M, a.top_k, a.H, a.out, s);
  }
  switch (chunks_per_lane(a.I)) {
    case 1: launch_w2<1>(a, s); break;
    case 2: launch_w2<2>(a, s); break;
    case 3: launch_w2<3>(a, s); break;
    default: launch_w2<4>(a, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe_host
