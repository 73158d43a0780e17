// moe_align: the two index lists of the grouped GEMMs.
// Page "Mixture of Experts in vLLM - From First Principles to fused_moe",
// section "How vLLM runs the layer: two index lists and no copies",
// sub-section "The two index lists": pair ids sorted by expert, each group
// padded with the id P = M*top_k to a multiple of BLOCK_SIZE_M, one expert
// per block.  The page leaves the order inside a group open; these kernels
// fix it to ascending pair id, which makes the result deterministic.
//
// The pairs are cut into G contiguous segments, one per workgroup of 16
// waves, and each segment into 16 contiguous wave pieces.  Counting uses a
// ballot per expert-id bit: the lanes of a 64-pair chunk that hold the same
// expert form one group (AND of matching ballots), so a chunk costs one LDS
// atomic per distinct expert rather than one per pair, and a pair's rank
// among the earlier pairs of its chunk with the same expert is a popcount.
//
//   G > 1:  align_count writes each segment's per-expert counts to scratch;
//           align_scatter then, in every workgroup, rebuilds the per-expert
//           block offsets (exclusive scan over experts), the start of its
//           own segment inside each expert group, recounts its segment per
//           wave, and scatters its pairs stably.
//   G == 1: align_scatter alone (counts come from its own segment).
// Block experts and pad entries are then filled by all workgroups.
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kTopkWaves = 4;   // tokens per workgroup of the fused top-k + align

// Lanes of the wave whose (valid) id equals this lane's id (ids < 512).
// All nine bit ballots are taken, whatever E: a bit above E's range is zero
// in every valid id and leaves the match unchanged.  The compares are all
// issued before the masks are combined, so the vector-to-scalar latency is
// paid once.
__device__ __forceinline__ unsigned long long match_lanes(int id, bool valid) {
  constexpr int kIdBits = 9;
  unsigned long long bb[kIdBits];
  const unsigned long long m0 = __ballot(valid);
#pragma unroll
  for (int b = 0; b < kIdBits; ++b) bb[b] = __ballot(valid && ((id >> b) & 1));
  __builtin_amdgcn_sched_group_barrier(0x2, kIdBits + 1, 0);   // the compares first
  unsigned long long m = m0;
#pragma unroll
  for (int b = 0; b < kIdBits; ++b) m &= ((id >> b) & 1) ? bb[b] : ~bb[b];
  return m;
}

// Count the experts of pairs [s0, s1) into hist[E] (LDS), one wave.
__device__ __forceinline__ void count_piece(const int32_t* __restrict__ ids, int s0, int s1,
                                            int* hist) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  // the next chunk's id is loaded before this chunk's ballots
  int id_next = s0 + lane < s1 ? ids[s0 + lane] : 0;
  for (int base = s0; base < s1; base += 64) {
    const int p = base + lane;
    const bool valid = p < s1;
    const int id = id_next;
    id_next = ids[min(p + 64, s1 - 1)];   // unconditional: one load in flight, no branch
    const unsigned long long m = match_lanes(id, valid);
    if (valid && (m & below) == 0ull) atomicAdd(&hist[id], __popcll(m));
  }
}

// Inclusive sum over the lanes of a wave with DPP (no LDS): Hillis-Steele
// shifts inside each 16-lane row, then row 0's total into row 1 and row 2's
// into row 3, then the total of rows 0-1 into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);    // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);    // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);    // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);    // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

__device__ __forceinline__ int block_scan_exclusive(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_inclusive_sum(v);
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

struct Seg {
  int s0, s1;   // this workgroup's pairs
  int w0, w1;   // this wave's pairs
};

__device__ __forceinline__ Seg segment(int P, int G, int gid) {
  Seg s;
  const int seg = ceil_div(ceil_div(P, G), 64) * 64;
  s.s0 = min(P, gid * seg);
  s.s1 = min(P, s.s0 + seg);
  const int piece = ceil_div(ceil_div(s.s1 - s.s0, kWaves), 64) * 64;
  const int w = threadIdx.x >> 6;
  s.w0 = min(s.s1, s.s0 + w * piece);
  s.w1 = min(s.s1, s.w0 + piece);
  return s;
}

// grid G (> 1): per-segment expert counts -> seg_counts[G][E]
__global__ __launch_bounds__(kThreads) void align_count_kernel(
    const int32_t* __restrict__ ids, int P, int E, int G, int32_t* __restrict__ seg_counts) {
  extern __shared__ int hist[];   // [E]
  for (int i = threadIdx.x; i < E; i += kThreads) hist[i] = 0;
  __syncthreads();
  const Seg sg = segment(P, G, blockIdx.x);
  count_piece(ids, sg.w0, sg.w1, hist);
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kThreads)
    seg_counts[(size_t)blockIdx.x * E + i] = hist[i];
}

// Segment gid of G of the index-list build (1024 threads; smem holds
// align_smem_ints(E) ints).  ids may live in global memory or in LDS.
// G == 1: counts come from this workgroup's own pass; G > 1: from
// seg_counts written by align_count_kernel.
__device__ __forceinline__ void align_segment(const int32_t* ids, int P, int E, int B, int G, int gid,
                              const int32_t* __restrict__ seg_counts,
                              int32_t* __restrict__ sorted, int32_t* __restrict__ expert_ids,
                              int32_t* __restrict__ boff_out, int32_t* __restrict__ counts_out,
                              int* smem) {
  int* hist = smem;                  // [kWaves][E] counts, then running positions
  int* boff = hist + kWaves * E;     // [E + 1]
  int* cnt = boff + E + 1;           // [E]
  int* wave_tot = cnt + E;           // [kWaves]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;

  for (int i = tid; i < kWaves * E; i += kThreads) hist[i] = 0;
  __syncthreads();
  const Seg sg = segment(P, G, gid);
  count_piece(ids, sg.w0, sg.w1, hist + w * E);
  __syncthreads();

  // expert totals, block offsets, start of every (wave, expert) run; each
  // expert's 16 wave counts are read once, all in flight together
  int wc[kWaves];
#pragma unroll
  for (int i = 0; i < kWaves; ++i) wc[i] = tid < E ? hist[i * E + tid] : 0;
  int n_e = 0, before = 0;
  if (tid < E) {
    if (G > 1) {
      // 16 independent loads in flight per batch: the counts were written
      // by another launch, so each is a trip past this XCD's L2
      for (int i0 = 0; i0 < G; i0 += 16) {
        int c[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) c[j] = seg_counts[(size_t)min(i0 + j, G - 1) * E + tid];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int v = i0 + j < G ? c[j] : 0;
          n_e += v;
          if (i0 + j < gid) before += v;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kWaves; ++i) n_e += wc[i];
    }
  }
  const int nb = tid < E ? ceil_div(n_e, B) : 0;
  int total_blocks = 0;
  const int excl = block_scan_exclusive(nb, wave_tot, total_blocks);
  if (tid < E) {
    boff[tid] = excl;
    cnt[tid] = n_e;
    if (gid == 0) {
      boff_out[tid] = excl;
      if (counts_out != nullptr) counts_out[tid] = n_e;
    }
    int run = excl * B + before;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      hist[i * E + tid] = run;
      run += wc[i];
    }
  }
  if (tid == 0) {
    boff[E] = total_blocks;
    if (gid == 0) boff_out[E] = total_blocks;
  }
  __syncthreads();

  // stable scatter, 64 pairs at a time per wave, in pair order
  const unsigned long long below = (1ull << lane) - 1ull;
  int* my_start = hist + w * E;
  int id_next = sg.w0 + lane < sg.w1 ? ids[sg.w0 + lane] : 0;
  for (int base = sg.w0; base < sg.w1; base += 64) {
    const int p = base + lane;
    const bool valid = p < sg.w1;
    const int id = id_next;
    id_next = ids[min(p + 64, sg.w1 - 1)];
    const unsigned long long match = match_lanes(id, valid);
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

  // expert of each block and the pad entries: one group of lanes per expert
  // (16 lanes for blocks of up to 16 pairs, else 32 or the whole wave; the
  // groups of all workgroups' waves share the experts), its lanes striding
  // over the expert's blocks and over the pad slots after its last pair
  const int glanes = B <= 16 ? 16 : (B <= 32 ? 32 : 64);
  const int gpw = 64 / glanes;
  const int gl = lane & (glanes - 1);
  const int gw = (gid * kWaves + w) * gpw + lane / glanes, nw = G * kWaves * gpw;
  for (int e = gw; e < E; e += nw) {
    const int b0 = boff[e], b1 = boff[e + 1];
    for (int blk = b0 + gl; blk < b1; blk += glanes) expert_ids[blk] = e;
    for (int pos = b0 * B + cnt[e] + gl; pos < b1 * B; pos += glanes) sorted[pos] = P;
  }
}

// grid G: offsets, stable scatter of this segment, block experts and pads.
__global__ __launch_bounds__(kThreads) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, int B, int G,
    const int32_t* __restrict__ seg_counts, int32_t* __restrict__ sorted,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ boff_out,
    int32_t* __restrict__ counts_out) {
  extern __shared__ int smem[];
  align_segment(ids, P, E, B, G, blockIdx.x, seg_counts, sorted, expert_ids, boff_out,
                counts_out, smem);
}

// Small batches (one align segment): top-k, one wave per token on the first
// kTopkWaves waves of each workgroup (one per SIMD, so tokens do not queue
// behind each other), then the index lists built by the workgroup that
// arrives last.  Each workgroup publishes its expert ids with agent-coherent
// stores, waits for them, and counts its arrival in *arrivals (zeroed by the
// router-logits kernel on the same stream) with an agent-scope
// acquire-release add; the last one reads all P ids back with
// agent-coherent loads.  A lone workgroup keeps its ids in LDS.  With qx
// set, each workgroup also writes the MXFP8 codes of its tokens' x rows.
__global__ __launch_bounds__(kThreads) void route_topk_align_kernel(
    const float* __restrict__ logits, int M, int E, int top_k, int renormalize, int B,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights,
    int32_t* __restrict__ sorted, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ boff_out, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ arrivals, const uint16_t* __restrict__ x, int H,
    uint8_t* __restrict__ qx, uint8_t* __restrict__ qxs) {
  extern __shared__ __attribute__((aligned(16))) int smem[];
  __shared__ int s_last;
  const int P = M * top_k;
  if (qx != nullptr) {
    // the MXFP8 layer's GEMM 1 input: codes and scales of this workgroup's
    // tokens' x rows (page "Mixture of Experts in vLLM ...", sub-section
    // "The two index lists": qhidden)
    const long long nb = H / 32;
    const long long b0 = (long long)blockIdx.x * kTopkWaves * nb;
    const long long b1 = (long long)min(M, ((int)blockIdx.x + 1) * kTopkWaves) * nb;
    for (long long b = b0 + threadIdx.x; b < b1; b += kThreads) mx_quantize_block(x, H, b, qx, qxs);
  }
  int* ids_lds = smem + align_smem_ints(E);
  float* tk = reinterpret_cast<float*>(smem + ((align_smem_ints(E) + P + 3) & ~3));
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + w;
  if (w < kTopkWaves && t < M) {
    const TopkSlot r =
        topk_token(logits + (size_t)t * E, E, top_k, renormalize, tk + w * topk_wave_floats(E));
    if (lane < top_k) {
      const size_t p = (size_t)t * top_k + lane;
      __hip_atomic_store(topk_ids + p, r.id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      topk_weights[p] = r.w;
      ids_lds[p] = r.id;
    }
  }
  if (gridDim.x > 1) {
    // Every wave's id stores have completed before the workgroup barrier;
    // the arrival is an agent-scope acquire-release add, so each workgroup's
    // stores happen before its arrival, and the last arrival (which then
    // reads every workgroup's ids) happens after all of them.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(arrivals, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
               (int)gridDim.x - 1;
    __syncthreads();
    if (!s_last) return;
    for (int i = threadIdx.x; i < P; i += kThreads)
      ids_lds[i] = __hip_atomic_load(topk_ids + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  align_segment(ids_lds, P, E, B, 1, 0, nullptr, sorted, expert_ids, boff_out, counts_out, smem);
}

}  // namespace

namespace moe_host {

constexpr size_t route_topk_align_lds(int P, int E) {
  return sizeof(int) *
         (size_t)(((align_smem_ints(E) + P + 3) & ~3) + kTopkWaves * topk_wave_floats(E));
}
// largest dynamic LDS of the fused launch: one full segment, 512 experts
constexpr size_t kFusedRouteMaxLds = route_topk_align_lds(kAlignPairsPerSegment, 512);
static_assert(kFusedRouteMaxLds <= 100 * 1024, "fused top-k + align LDS");

hipError_t launch_route_topk_align(const RouteArgs& r, const AlignArgs& a, int32_t* arrivals,
                                   hipStream_t s) {
  const size_t lds = route_topk_align_lds(r.M * r.top_k, r.E);
  static bool lds_set[kMaxDevices] = {};
  const hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(&route_topk_align_kernel),
                                            (int)kFusedRouteMaxLds, lds_set);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_topk_align_kernel, dim3(ceil_div_host(r.M, kTopkWaves)), dim3(kThreads),
                     lds, s, r.logits, r.M, r.E, r.top_k, r.renormalize, a.block_m, r.topk_ids,
                     r.topk_weights, a.sorted_token_ids, a.expert_ids, a.expert_block_offsets,
                     a.expert_counts, arrivals, r.x, r.H, r.qx_codes, r.qx_scales);
  return hipGetLastError();
}

int align_segments(int P) {
  const int g = (P + kAlignPairsPerSegment - 1) / kAlignPairsPerSegment;
  return g < 1 ? 1 : (g > kAlignMaxSegments ? kAlignMaxSegments : g);
}

size_t align_scratch_bytes(int P, int E) {
  const int G = align_segments(P);
  return G > 1 ? (size_t)G * E * sizeof(int32_t) : 0;
}

hipError_t launch_align(const AlignArgs& a, hipStream_t s) {
  const int G = align_segments(a.P);
  if (G > 1) {
    hipLaunchKernelGGL(align_count_kernel, dim3(G), dim3(kThreads), sizeof(int) * a.E, s,
                       a.topk_ids, a.P, a.E, G, a.scratch);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const size_t lds = sizeof(int) * (size_t)align_smem_ints(a.E);
  hipLaunchKernelGGL(align_scatter_kernel, dim3(G), dim3(kThreads), lds, s, a.topk_ids, a.P,
                     a.E, a.block_m, G, a.scratch, a.sorted_token_ids, a.expert_ids,
                     a.expert_block_offsets, a.expert_counts);
  return hipGetLastError();
}

}  // namespace moe_host
