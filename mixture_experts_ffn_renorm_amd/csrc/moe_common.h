// Internal helpers shared by the HIP kernels of the MoE layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// 16-byte payload moved by one global_load_dwordx4 / ds_read_b128.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// D = A(16x32) * B(32x16) + C on the CDNA4 matrix core, bf16 in, fp32 out.
// Operand layout (one 16x16 tile, lane l in 0..63):
//   A: lane l holds row (l % 16), k = 8*(l / 16) .. 8*(l / 16) + 7
//   B: lane l holds column (l % 16), the same 8 k values
//   C: lane l holds column (l % 16), rows 4*(l / 16) .. 4*(l / 16) + 3
// Only the pairing of A and B k values matters for the sum, so callers may
// map those 32 "k slots" to any 32 distinct k indices as long as A and B
// use the same map.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// SiLU(g) * u with SiLU(g) = g / (1 + exp(-g)).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Zero-filled 16-byte load when `ok` is false.
__device__ __forceinline__ u32x4 load16_or_zero(const void* p, bool ok) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (ok) v = *reinterpret_cast<const u32x4*>(p);
  return v;
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---- global -> LDS copies (global_load_lds_dwordx4) ----
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

// 16 zero bytes that out-of-range lanes copy instead of real data.
static __device__ __attribute__((aligned(16))) const uint32_t kZeroPage[4] = {0u, 0u, 0u, 0u};

// Cache policy of a copy: 0 = default, kNonTemporal = streamed once.
constexpr int kNonTemporal = 2;

// Each lane copies 16 bytes from `src` to LDS at lds_dst + 16 * lane
// (lds_dst must be the same for the whole wave).
template <int kPolicy = 0>
__device__ __forceinline__ void load_lds16(const void* src, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)lds_dst, 16, 0, kPolicy);
}

// Waits until at most N vector-memory operations of this wave are pending.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  // gfx9 s_waitcnt encoding: vmcnt = bits 3:0 and 15:14; expcnt (6:4) and
  // lgkmcnt (11:8) left at their maxima, i.e. not waited on.
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence (a fenced barrier also waits for
// every copy still in flight).  The empty asm statements keep the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wave-wide reductions over 64 lanes.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// Sum of the top_k fp32 partial rows of one token at one column, in slot
// order, read with agent-coherent loads (rows written by other workgroups).
// All loads are issued before the first add.
__device__ __forceinline__ float sum_partials(const float* src, int stride, int top_k) {
  constexpr int kMaxK = 32;
  float v[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < top_k)
      v[j] = __hip_atomic_load(src + (size_t)j * stride, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < top_k) sum += v[j];
  return sum;
}

// Workgroups are handed to the 8 XCDs of the chip round-robin (id % 8).
// Map a linear workgroup id to a logical tile id so that every XCD works on
// one contiguous range of logical tiles (tiles that share operands then
// share an L2).  `n` = real tile count; returns -1 for ids without a tile.
__device__ __forceinline__ int xcd_contiguous_tile(int wg, int n) {
  const int chunk = (n + 7) >> 3;
  const int xcd = wg & 7, slot = wg >> 3;
  if (slot >= chunk) return -1;
  const int t = xcd * chunk + slot;
  return t < n ? t : -1;
}

}  // namespace moe

// Host-side launchers (defined in the kernel sources, used by the C ABI).
namespace moe_host {

inline int ceil_div_host(int a, int b) { return (a + b - 1) / b; }

struct RouteArgs {
  const uint16_t* x;
  const uint16_t* w_router;
  const float* bias;
  int M, H, E, top_k, renormalize;
  float* logits;        // [M, E] scratch or caller output
  int32_t* topk_ids;    // [M, top_k]
  float* topk_weights;  // [M, top_k]
  float* zero_ptr;      // optional region to clear (combine arrival counters)
  size_t zero_words;    // number of 4-byte words to clear
};
hipError_t launch_route_logits(const RouteArgs& a, hipStream_t s);
hipError_t launch_route_topk(const RouteArgs& a, hipStream_t s);

struct AlignArgs {
  const int32_t* topk_ids;
  int P, E, block_m;
  int32_t* sorted_token_ids;
  int32_t* expert_ids;
  int32_t* expert_block_offsets;
  int32_t* expert_counts;  // may be null
  int32_t* scratch;        // align_scratch_bytes(P, E) bytes (null when 0)
};
constexpr int kAlignPairsPerSegment = 2048;  // pairs per align workgroup
constexpr int kAlignMaxSegments = 64;
int align_segments(int P);
size_t align_scratch_bytes(int P, int E);
hipError_t launch_align(const AlignArgs& a, hipStream_t s);

struct GemmArgs {
  const uint16_t* a_src;     // GEMM 1: x [M, H]; GEMM 2: act [P, I]
  const uint16_t* w;         // GEMM 1: w13 [E, 2I, H]; GEMM 2: w2 [E, H, I]
  const int32_t* sorted_token_ids;
  const int32_t* expert_ids;
  const int32_t* expert_block_offsets;
  const float* topk_weights; // GEMM 2 only
  int M, top_k, E, H, I, block_m, max_blocks;
  uint16_t* out;             // GEMM 1: act [P, I]; GEMM 2: out [M, H]
  float* partial;            // GEMM 2: fp32 weighted partial rows [P, H]
  int32_t* counters;         // GEMM 2: arrival counters [M, ceil(H/64)] (zeroed)
};
hipError_t launch_gemm1_tiled(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm2_tiled(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm1_stream(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm2_stream(const GemmArgs& a, hipStream_t s);
hipError_t launch_fill_zero(float* p, size_t words, hipStream_t s);

// Tile constants the host needs for grids and counters.
constexpr int kTiledBK = 64;
constexpr int kTiledG1Features = 128;   // act columns per GEMM 1 tile (128 gate + 128 up rows)
constexpr int kTiledG2Features = 256;   // output columns per GEMM 2 tile
constexpr int kStreamG1Features = 16;   // act columns per streaming GEMM 1 tile
constexpr int kStreamG2Features = 32;   // output columns per streaming GEMM 2 tile
constexpr int kStreamBK = 256;          // K elements per streaming LDS slice
constexpr int kCounterCols = 32;        // combine counters: room for one per (token, 32 columns)

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace moe_host
