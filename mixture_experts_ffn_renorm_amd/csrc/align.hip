// moe_align: the two index lists of the grouped GEMMs.
// Page "Mixture of Experts in vLLM - From First Principles to fused_moe",
// section "How vLLM runs the layer: two index lists and no copies",
// sub-section "The two index lists": pair ids sorted by expert, each group
// padded with the id P = M*top_k to a multiple of BLOCK_SIZE_M, one expert
// per block.  The page leaves the order inside a group open; this kernel
// fixes it to ascending pair id, which makes the result deterministic.
//
// One workgroup of 16 waves does the whole job in LDS:
//   1. each wave counts the experts of one contiguous segment of pairs into
//      its own LDS histogram;
//   2. per expert: n_e, blocks ceil(n_e / B), exclusive scan over experts
//      -> block offsets; per (wave, expert) start position = expert start +
//      pairs of that expert in earlier segments;
//   3. stable scatter: each wave walks its segment 64 pairs at a time; a
//      pair's rank among earlier lanes with the same expert comes from a
//      ballot per id bit (AND of matching ballots) and a popcount;
//   4. expert id of every block and the pad entries (binary search of the
//      block offsets).
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;

__device__ __forceinline__ int block_scan_exclusive(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int t = wave_tot[i];
    if (i < w) base += t;
    total += t;
  }
  return base + incl - v;
}

// Largest e with boff[e] <= blk; for blk < num_blocks that expert is never
// empty (an empty expert e has boff[e] == boff[e+1], so e+1 also qualifies).
__device__ __forceinline__ int expert_of_block(const int* boff, int E, int blk) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (boff[mid] <= blk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) void align_kernel(
    const int32_t* __restrict__ ids, int P, int E, int B, int32_t* __restrict__ sorted,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ boff_out,
    int32_t* __restrict__ counts_out) {
  extern __shared__ int smem[];
  int* hist = smem;                   // [kWaves][E]  counts, then running positions
  int* boff = hist + kWaves * E;      // [E + 1]
  int* cnt = boff + E + 1;            // [E]
  int* wave_tot = cnt + E;            // [kWaves]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  for (int i = tid; i < kWaves * E; i += kThreads) hist[i] = 0;
  __syncthreads();

  // 1. per-wave histograms of contiguous segments (segment length multiple of 64)
  const int seg = ceil_div(ceil_div(P, kWaves), 64) * 64;
  const int s0 = min(P, w * seg), s1 = min(P, s0 + seg);
  for (int p = s0 + lane; p < s1; p += 64) atomicAdd(&hist[w * E + ids[p]], 1);
  __syncthreads();

  // 2. counts, block offsets, per-(wave, expert) start positions
  int n_e = 0, nb = 0;
  if (tid < E) {
    for (int i = 0; i < kWaves; ++i) n_e += hist[i * E + tid];
    nb = ceil_div(n_e, B);
  }
  int total_blocks = 0;
  const int excl = block_scan_exclusive(nb, wave_tot, total_blocks);
  if (tid < E) {
    boff[tid] = excl;
    cnt[tid] = n_e;
    boff_out[tid] = excl;
    if (counts_out != nullptr) counts_out[tid] = n_e;
    int run = excl * B;
    for (int i = 0; i < kWaves; ++i) {
      const int c = hist[i * E + tid];
      hist[i * E + tid] = run;
      run += c;
    }
  }
  if (tid == 0) {
    boff[E] = total_blocks;
    boff_out[E] = total_blocks;
  }
  __syncthreads();

  // 3. stable scatter, 64 pairs at a time per wave, in pair order
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  int* my_start = hist + w * E;
  for (int base = s0; base < s1; base += 64) {
    const int p = base + lane;
    const bool valid = p < s1;
    const int id = valid ? ids[p] : 0;
    unsigned long long match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (id >> b) & 1;
      const unsigned long long bb = __ballot(valid && bit);
      match &= bit ? bb : ~bb;
    }
    const int rank = __popcll(match & below);
    const int size = __popcll(match);
    int pos = 0;
    if (valid) pos = my_start[id] + rank;
    // every lane has read its start before the group's last lane moves it on
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      sorted[pos] = p;
      if (rank == size - 1) my_start[id] = pos + 1;
    }
    __builtin_amdgcn_wave_barrier();
  }

  // 4. expert of each block, pad entries
  for (int blk = tid; blk < total_blocks; blk += kThreads)
    expert_ids[blk] = expert_of_block(boff, E, blk);
  const int nslots = total_blocks * B;
  for (int pos = tid; pos < nslots; pos += kThreads) {
    const int blk = pos / B;
    const int e = expert_of_block(boff, E, blk);
    if (pos - boff[e] * B >= cnt[e]) sorted[pos] = P;
  }
}

}  // namespace

namespace moe_host {

hipError_t launch_align(const AlignArgs& a, hipStream_t s) {
  const size_t lds = sizeof(int) * ((size_t)kWaves * a.E + (a.E + 1) + a.E + kWaves);
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kThreads), lds, s, a.topk_ids, a.P, a.E,
                     a.block_m, a.sorted_token_ids, a.expert_ids, a.expert_block_offsets,
                     a.expert_counts);
  return hipGetLastError();
}

}  // namespace moe_host
