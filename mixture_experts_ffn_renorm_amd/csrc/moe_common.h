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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values to packed bf16 (lo in the low half), round to nearest
// even, NaN stays NaN: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
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

// Waits until this wave's LDS operations have completed (vmcnt and expcnt
// left at their maxima, i.e. not waited on).
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Workgroup barrier without a memory fence (a fenced barrier also waits for
// every copy still in flight).  The empty asm statements keep the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- MXFP8 (OCP microscaling: E8M0 scale per 32 values, E4M3 elements) ----

// The nearest E4M3 magnitude to a >= 0, ties to the even code, saturated at
// 448: steps of 2^-9 below 2^-6 (subnormals), 3 mantissa bits above.
__device__ __forceinline__ float e4m3_round_mag(float a) {
  const float sub = __builtin_rintf(a * 512.f) * (1.f / 512.f);
  uint32_t u = __float_as_uint(a);
  u = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;   // drop 20 bits, ties to even
  const float r = a < 0.015625f ? sub : __uint_as_float(u);
  return r < 448.f ? r : 448.f;
}

// E4M3 magnitude code (7 bits) of an exactly representable magnitude r.
__device__ __forceinline__ uint32_t e4m3_code_of_mag(float r) {
  if (r < 0.015625f) return (uint32_t)(r * 512.f);        // subnormal codes 0..7
  const uint32_t u = __float_as_uint(r);
  return ((((u >> 23) & 0xFFu) - 120u) << 3) | ((u >> 20) & 7u);
}

// Shared exponent of a block whose largest magnitude is amax: floor(log2
// amax) - 8 (8 = the exponent of E4M3's largest power of two), clamped to
// E8M0's range [-127, 127]; -127 for a zero or subnormal amax.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  const int s = ef == 0 ? -127 : ef - 127 - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// E4M3 byte of v * 2^-shared (nearest, ties to even, saturated, sign kept).
__device__ __forceinline__ uint32_t e4m3_of(float v, int shared) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  return sign | e4m3_code_of_mag(e4m3_round_mag(__builtin_ldexpf(__builtin_fabsf(v), -shared)));
}

// Block b (32 values) of the bf16 rows src [rows, K] into E4M3 codes and its
// E8M0 scale byte (K % 32 == 0; src and codes 16-byte aligned).
__device__ __forceinline__ void mx_quantize_block(const uint16_t* __restrict__ src, int K,
                                                  long long b, uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  const int nb = K / 32;
  const long long row = b / nb;
  const int blk = (int)(b - row * nb);
  const size_t base = (size_t)row * K + (size_t)blk * 32;
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src + base);
  u32x4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = s4[i];
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = bf16_lo(w[i][j]);
      v[8 * i + 2 * j + 1] = bf16_hi(w[i][j]);
    }
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  const int shared = mx_shared_exp(amax);
  u32x4 out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i0 = 16 * h + 4 * j;
      out[h][j] = e4m3_of(v[i0], shared) | (e4m3_of(v[i0 + 1], shared) << 8) |
                  (e4m3_of(v[i0 + 2], shared) << 16) | (e4m3_of(v[i0 + 3], shared) << 24);
    }
  u32x4* d4 = reinterpret_cast<u32x4*>(codes + base);
  d4[0] = out[0];
  d4[1] = out[1];
  scales[b] = (uint8_t)(shared + 127);
}

// Wave-wide reductions over 64 lanes.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
  return v;
}
// The sum runs on DPP (no LDS round trips): Hillis-Steele shifts inside each
// 16-lane row, then row 0's total into row 1 and row 2's into row 3, then
// rows 0-1 into rows 2 and 3; lane 63 ends with the total, which every lane
// reads.  A fixed order: bitwise repeatable.
template <int kCtrl, int kRowMask, bool kBound>
__device__ __forceinline__ float dpp_shifted_add(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xf, kBound);
  return v + __builtin_bit_cast(float, s);
}
// Sum over each group of kLanes consecutive lanes (16, 32 or 64), valid in
// the group's last lane.
template <int kLanes>
__device__ __forceinline__ float group_sum_last(float v) {
  static_assert(kLanes == 16 || kLanes == 32 || kLanes == 64, "lane group");
  v = dpp_shifted_add<0x111, 0xf, true>(v);    // row_shr:1
  v = dpp_shifted_add<0x112, 0xf, true>(v);    // row_shr:2
  v = dpp_shifted_add<0x114, 0xf, true>(v);    // row_shr:4
  v = dpp_shifted_add<0x118, 0xf, true>(v);    // row_shr:8
  if (kLanes >= 32) v = dpp_shifted_add<0x142, 0xa, false>(v);   // row_bcast:15
  if (kLanes == 64) v = dpp_shifted_add<0x143, 0xc, false>(v);   // row_bcast:31
  return v;
}
// Maximum over each 16-lane row, in every lane of the row (DPP: swap
// neighbours, swap pairs, mirror each half row, mirror the row).
template <int kCtrl>
__device__ __forceinline__ float dpp_max_with(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, false);
  return __builtin_fmaxf(v, __builtin_bit_cast(float, s));
}
__device__ __forceinline__ float row16_max(float v) {
  v = dpp_max_with<0xb1>(v);    // quad_perm [1, 0, 3, 2]
  v = dpp_max_with<0x4e>(v);    // quad_perm [2, 3, 0, 1]
  v = dpp_max_with<0x141>(v);   // row_half_mirror
  v = dpp_max_with<0x140>(v);   // row_mirror
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum_last<64>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
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

// LDS ints used by the index-list build of one segment (1024 threads).
__host__ __device__ constexpr int align_smem_ints(int E) { return 16 * E + (E + 1) + E + 16; }

// Per-wave LDS floats of topk_token.  E <= 128: 32 slot ids and 32 slot
// weights.  Larger E: all logits padded to a multiple of 64 (only for the
// many-ties path), 64 lane maxima, 64 candidate logits, 64 candidate ids,
// 32 slot ids, 32 slot logits.
__host__ __device__ constexpr int topk_wave_floats(int E) {
  return E <= 128 ? 64 : ((E + 63) & ~63) + 256;
}

struct TopkSlot {
  int id;     // expert of slot lane (lane < top_k)
  float w;    // its routing weight
};

namespace topk_detail {
// Order-preserving 32-bit key of a finite logit (or -inf): larger logit,
// larger key; -0 and +0 get the same key, as they compare equal.  Real keys
// are >= 0x007fffff (that of -inf), so 0 marks an empty slot.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// Number of the wave's keys >= c (uniform).  All compares are issued
// before the first population count (each ballot lands in its own scalar
// register pair), so the vector-to-scalar latency is paid once per count,
// not once per ballot.
template <int NB>
__device__ __forceinline__ int count_ge(const uint32_t (&key)[NB], uint32_t c) {
  unsigned long long m[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) m[i] = __ballot(key[i] >= c);
  __builtin_amdgcn_sched_group_barrier(0x2, NB, 0);       // the compares (VALU)
  __builtin_amdgcn_sched_group_barrier(0x4, 2 * NB, 0);   // then the counts (SALU)
  int n = 0;
#pragma unroll
  for (int i = 0; i < NB; ++i) n += __popcll(m[i]);
  return n;
}

// topk_token for E <= 64 NB (NB <= 2); lane l holds logits l, l + 64, ...
template <int NB>
__device__ __forceinline__ TopkSlot topk_nb(const float* __restrict__ row, int E, int top_k,
                                            int renormalize, float* scratch) {
  const int lane = threadIdx.x & 63;
  int* s_id = reinterpret_cast<int*>(scratch);   // [32]
  float* s_w = scratch + 32;                     // [32]
  float v[NB];
  uint32_t key[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : 0.f;
    key[i] = e < E ? order_key(v[i]) : 0u;
  }
  // T = the top_k-th largest key: the largest value whose count of keys at
  // or above it is still >= top_k, built one bit at a time from the top.
  uint32_t T = 0u;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    if (count_ge(key, c) >= top_k) T = c;
  }
  // kept: every key above T, then keys equal to T in expert order until
  // top_k are kept (exact ties go to the lower expert id)
  int need = top_k - count_ge(key, T + 1u);
  const unsigned long long below = (1ull << lane) - 1ull;
  bool kept[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const unsigned long long eq = __ballot(key[i] == T);
    kept[i] = key[i] > T || (key[i] == T && __popcll(eq & below) < need);
    need -= min(__popcll(eq), need);
  }
  // slot of a kept expert = kept experts with a larger logit, or the same
  // logit and a lower id; the largest kept key is the softmax shift
  int slot[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) slot[i] = 0;
  uint32_t kmax = 0u;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    for (unsigned long long m = __ballot(kept[j]); m != 0ull; m &= m - 1ull) {
      const int L = __builtin_ctzll(m);
      const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)key[j], L);
      const int idj = 64 * j + L;
      kmax = kj > kmax ? kj : kmax;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        slot[i] += (kj > key[i]) | ((kj == key[i]) & (idj < lane + 64 * i));
    }
  }
  const float mx = key_logit(kmax);
  float ex[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) ex[i] = __expf(v[i] - mx);
  float denom = 0.f;
  if (renormalize) {
    // the softmax denominator cancels: sum the kept exponentials, in expert order
#pragma unroll
    for (int j = 0; j < NB; ++j)
      for (unsigned long long m = __ballot(kept[j]); m != 0ull; m &= m - 1ull)
        denom += __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex[j]), __builtin_ctzll(m)));
  } else {
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (lane + 64 * i < E) ps += ex[i];
    denom = wave_sum(ps);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i)
    if (kept[i]) {
      s_id[slot[i]] = lane + 64 * i;
      s_w[slot[i]] = ex[i] / denom;
    }
  __builtin_amdgcn_wave_barrier();
  TopkSlot out{0, 0.f};
  if (lane < top_k) {
    out.id = s_id[lane];
    out.w = s_w[lane];
  }
  __builtin_amdgcn_wave_barrier();   // scratch may be reused by the next token
  return out;
}

// Adds to r the count of the 16 values at o that beat v: kMode 0 counts
// o >= v (all of them precede v's own position), 1 counts o > v (all follow
// it), 2 counts o > v plus equal values at lower positions (jbase + u < own).
template <int kMode>
__device__ __forceinline__ int count16(const float* o, float v, int jbase, int own, int r) {
  const f32x4* q = reinterpret_cast<const f32x4*>(o);
  f32x4 c[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) c[u] = q[u];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int z = 0; z < 4; ++z) {
      const float x = c[u][z];
      if (kMode == 0) r += x >= v;
      if (kMode == 1) r += x > v;
      if (kMode == 2) r += (x > v) | ((x == v) & (jbase + 4 * u + z < own));
    }
  return r;
}

// Rank of v (at position own) among the n values at o, n a multiple of 64
// padded with -inf: larger values plus equal values at lower positions.
__device__ __forceinline__ int rank_in(const float* o, int n, float v, int own) {
  const int blk = own & ~63;
  int r = 0;
  for (int j = 0; j < blk; j += 16) r = count16<0>(o + j, v, j, own, r);
#pragma unroll
  for (int j = 0; j < 64; j += 16) r = count16<2>(o + blk + j, v, blk + j, own, r);
  for (int j = blk + 64; j < n; j += 16) r = count16<1>(o + j, v, j, own, r);
  return r;
}

// topk_token for E > 128.  Lane l owns logits l, l + 64, ...  The k-th
// largest of the 64 lane maxima T is a lower bound of the k-th largest
// logit (k lanes hold a value >= T), so the kept experts are among the
// candidates >= T, usually little more than k of them.  Candidates are
// packed in expert order (one ballot per 64-expert block) and each is ranked
// against the others with broadcast LDS reads (rank = larger logits + equal
// logits of lower id); rank j < k is slot j.  More than 64 candidates (many
// exact ties) ranks every logit the same way.  The max is slot 0.
__device__ inline TopkSlot topk_lanemax(const float* __restrict__ row, int E, int top_k,
                                        int renormalize, float* scratch) {
  constexpr int kMaxPerLane = 8;
  const int lane = threadIdx.x & 63;
  const int nblk = (E + 63) >> 6;
  float* lw = scratch;                                       // [64 nblk]
  float* lm = scratch + 64 * nblk;                           // [64]
  float* c_v = lm + 64;                                      // [64]
  int* c_id = reinterpret_cast<int*>(c_v + 64);              // [64]
  int* s_id = c_id + 64;                                     // [32]
  float* s_l = reinterpret_cast<float*>(s_id + 32);          // [32]
  float v[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
  }
  float lmax = v[0];
#pragma unroll
  for (int i = 1; i < kMaxPerLane; ++i) lmax = fmaxf(lmax, v[i]);
  lm[lane] = lmax;
  __builtin_amdgcn_wave_barrier();
  int gt = 0;
#pragma unroll
  for (int j = 0; j < 64; j += 16) gt = count16<1>(lm + j, lmax, j, lane, gt);
  const float T = -wave_max(gt < top_k ? -lmax : -INFINITY);

  // pack the candidates in expert order
  int C = 0;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    if (i >= nblk) break;
    const bool cand = lane + 64 * i < E && v[i] >= T;
    const unsigned long long m = __ballot(cand);
    const int pos = C + __popcll(m & below);
    if (cand && pos < 64) {
      c_v[pos] = v[i];
      c_id[pos] = lane + 64 * i;
    }
    C += __popcll(m);
  }
  if (C <= 64) {
    if (lane >= C) c_v[lane] = -INFINITY;
    __builtin_amdgcn_wave_barrier();
    const float my = c_v[lane];
    int r = 0;
    for (int j = 0; j < C; j += 16) r = count16<2>(c_v + j, my, j, lane, r);
    if (lane < C && r < top_k) {
      s_id[r] = c_id[lane];
      s_l[r] = my;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (i < nblk) lw[lane + 64 * i] = v[i];
    __builtin_amdgcn_wave_barrier();
    for (int i = 0; i < nblk; ++i) {
      const int e = lane + 64 * i;
      const float vi = lw[e];
      const int r = rank_in(lw, 64 * nblk, vi, e);
      if (e < E && r < top_k) {
        s_id[r] = e;
        s_l[r] = vi;
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  const float m = s_l[0];
  float denom;
  if (renormalize) {
    denom = 0.f;
    for (int q = 0; q < top_k; ++q) denom += __expf(s_l[q] - m);
  } else {
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (lane + 64 * i < E) ps += __expf(v[i] - m);
    denom = wave_sum(ps);
  }
  TopkSlot out{0, 0.f};
  if (lane < top_k) {
    out.id = s_id[lane];
    out.w = __expf(s_l[lane] - m) / denom;
  }
  __builtin_amdgcn_wave_barrier();   // scratch may be reused by the next token
  return out;
}
}  // namespace topk_detail

// Router steps for one token, by one wave (page "Mixture of Experts in vLLM
// - From First Principles to fused_moe", section "One expert, and one
// token", sub-section "One token uses only 8 experts"): softmax over all E
// logits, keep the top_k largest in descending order (exact ties -> lower
// expert id), rescale the kept probabilities to sum 1 if renormalize.
//
// E <= 128 (two logits a lane at most): each logit maps to an
// order-preserving 32-bit key, and the top_k-th largest key T is found by a
// 32-step bitwise search whose counts are wave ballots (no LDS, no
// shuffles).  The kept experts are the keys above T plus the lowest-id keys
// equal to T; each kept expert's slot is the number of kept experts that
// precede it (larger logit, or the same logit and a lower id), counted in a
// scalar loop over the kept set that reads each kept key once.  One LDS
// round trip moves each kept expert to its slot lane.  Larger E keeps the
// lane-maxima bound and LDS ranks (topk_lanemax), which measured faster
// there: the ballot count grows with the logits per lane.
//
// With renormalize the softmax denominator cancels and only the kept
// exponentials are summed; without it every lane adds its share and a wave
// sum follows.  E <= 512, top_k <= 32, finite logits.  Returns slot lane's
// expert and weight on lanes < top_k.
__device__ inline TopkSlot topk_token(const float* __restrict__ row, int E, int top_k,
                                      int renormalize, float* scratch) {
  if (E <= 64) return topk_detail::topk_nb<1>(row, E, top_k, renormalize, scratch);
  if (E <= 128) return topk_detail::topk_nb<2>(row, E, top_k, renormalize, scratch);
  return topk_detail::topk_lanemax(row, E, top_k, renormalize, scratch);
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
  float* zero_ptr;      // optional region to clear (arrival counter of the fused top-k + align)
  size_t zero_words;    // number of 4-byte words to clear
  uint8_t* qx_codes;    // optional: launch_route_topk also writes MXFP8 codes [M, H] of x
  uint8_t* qx_scales;   //           and their E8M0 scales [M, H/32] (H % 32 == 0)
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
// Top-k of all tokens and the index lists in one launch (one align segment);
// arrivals: one int, zero before the launch.
hipError_t launch_route_topk_align(const RouteArgs& r, const AlignArgs& a, int32_t* arrivals,
                                   hipStream_t s);

struct GemmArgs {
  const uint16_t* a_src;     // GEMM 1: x [M, H]; GEMM 2: act [P, I]
  const uint16_t* w;         // GEMM 1: w13 [E, 2I, H]; GEMM 2: w2 [E, H, I]
  const int32_t* sorted_token_ids;
  const int32_t* expert_ids;
  const int32_t* expert_block_offsets;
  const float* topk_weights; // GEMM 2 only
  int M, top_k, E, H, I, block_m, max_blocks;
  uint16_t* out;             // GEMM 1: act [P, I]; GEMM 2: out [M, H]
  float* partial;            // GEMM 2: pair-order rows [P, H], fp32 weighted
                             // (streaming) or bf16 (tiled)
  int mx;                    // tiled only: a_src and w hold MXFP8 E4M3 bytes
  const uint8_t* a_scales;   // MX: E8M0 per 32 k of each a_src row
  const uint8_t* w_scales;   // MX: E8M0 per 32 k of each weight row
};
// MXFP8 codes [rows, K] and E8M0 scales [rows, K/32] of bf16 rows (K % 32 == 0).
hipError_t launch_mx_quantize(const uint16_t* src, int rows, int K, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);
hipError_t launch_gemm1_tiled(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm2_tiled(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm1_stream(const GemmArgs& a, hipStream_t s);
// MXFP8 streaming GEMM 1 (block_m 16; a_src / a_scales: x codes and scales)
// that writes act already quantized: codes qact [P, I] and E8M0 scales
// sact [P, I/32] (I % 32 == 0, H % 128 == 0).
hipError_t launch_gemm1_stream_mx_quantize(const GemmArgs& a, uint8_t* qact, uint8_t* sact,
                                           hipStream_t s);
hipError_t launch_gemm2_stream(const GemmArgs& a, hipStream_t s);
// out[t] = bf16(sum over slots j of partial[t*top_k + j]), j ascending.
hipError_t launch_combine_partials(const float* partial, int M, int top_k, int H, uint16_t* out,
                                   hipStream_t s);

// Per-pair GEMVs of very small batches: GEMV 1 writes act [P, I]; GEMV 2
// multiplies, weights and sums each token's top_k rows straight into
// out [M, H] (sorted == null: pair p's expert is topk_ids[p]), or, with
// index lists of one pair per block (sorted, expert_ids from block_m 1),
// writes weighted fp32 rows to partial [P, H] and queues the per-token sum.
struct PairGemvArgs {
  const uint16_t* x;          // [M, H]
  const uint16_t* w13;        // [E, 2I, H]
  const uint16_t* w2;         // [E, H, I]
  const int32_t* topk_ids;    // [M, top_k] (no lists)
  const float* topk_weights;  // [M, top_k]
  int M, top_k, H, I;
  uint16_t* act;              // [M*top_k, I]
  uint16_t* out;              // [M, H]
  const int32_t* sorted;      // block_m 1 lists: pair of block b, or null
  const int32_t* expert_ids;  // block_m 1 lists: expert of block b
  float* partial;             // [M*top_k, H] fp32 (lists form of GEMV 2)
};
// Per-pair GEMVs on group-quantized expert weights (affine, 64-element
// groups, 4 or 8 bits): GEMV 1 writes act [P, I]; GEMV 2 multiplies,
// weights and sums each token's top_k rows into out [M, H].
struct QPairGemvArgs {
  const uint16_t* x;            // [M, H]
  const uint32_t* w13q;         // [E, 2I, H*bits/32] packed codes
  const uint16_t* w13_scales;   // [E, 2I, H/64] bf16
  const uint16_t* w13_biases;   // [E, 2I, H/64] bf16
  const uint32_t* w2q;          // [E, H, I*bits/32]
  const uint16_t* w2_scales;    // [E, H, I/64]
  const uint16_t* w2_biases;    // [E, H, I/64]
  const int32_t* topk_ids;      // [M, top_k]
  const float* topk_weights;    // [M, top_k]
  int M, top_k, H, I, bits;
  uint16_t* act;                // [M*top_k, I]
  uint16_t* out;                // [M, H]
};
// Per-pair GEMVs on MXFP8 expert weights: GEMV 1 reads the MXFP8 codes of x
// (written by the top-k launch) and writes act [P, I] bf16; GEMV 2 quantizes
// each act row to MXFP8 in registers, multiplies, weights and sums each
// token's top_k rows into out [M, H].  H, I multiples of 128.
struct MxPairGemvArgs {
  const uint8_t* qx;            // [M, H] E4M3
  const uint8_t* qx_scales;     // [M, H/32] E8M0
  const uint8_t* w13;           // [E, 2I, H] E4M3
  const uint8_t* w13_scales;    // [E, 2I, H/32]
  const uint8_t* w2;            // [E, H, I] E4M3
  const uint8_t* w2_scales;     // [E, H, I/32]
  const int32_t* topk_ids;      // [M, top_k]
  const float* topk_weights;    // [M, top_k]
  int M, top_k, H, I;
  uint16_t* act;                // [M*top_k, I]
  uint16_t* out;                // [M, H]
};
hipError_t launch_mx_pair_gemv1(const MxPairGemvArgs& a, hipStream_t s);
hipError_t launch_mx_pair_gemv2(const MxPairGemvArgs& a, hipStream_t s);

hipError_t launch_qpair_gemv1(const QPairGemvArgs& a, hipStream_t s);
hipError_t launch_qpair_gemv2(const QPairGemvArgs& a, hipStream_t s);

// Weight-streaming grouped GEMMs on group-quantized experts over index lists
// with block_m 16: GEMM 1 writes act [P, I]; GEMM 2 writes fp32 weighted
// pair-order rows into partial [P, H] and its per-token sum into out.
struct QGemmArgs {
  const uint16_t* x;            // [M, H]
  const uint32_t* w13q;         // [E, 2I, H*bits/32]
  const uint16_t* w13_scales;   // [E, 2I, H/64]
  const uint16_t* w13_biases;
  const uint32_t* w2q;          // [E, H, I*bits/32]
  const uint16_t* w2_scales;    // [E, H, I/64]
  const uint16_t* w2_biases;
  const int32_t* sorted_token_ids;
  const int32_t* expert_ids;
  const int32_t* expert_block_offsets;
  const float* topk_weights;    // [M*top_k]
  int M, top_k, E, H, I, bits, max_blocks;
  uint16_t* act;                // [M*top_k, I]
  float* partial;               // [M*top_k, H]
  uint16_t* out;                // [M, H]
};
// H and I multiples of 128
bool qgemm_stream_shapes_ok(int H, int I);
hipError_t launch_qgemm1_stream(const QGemmArgs& a, hipStream_t s);
hipError_t launch_qgemm2_stream(const QGemmArgs& a, hipStream_t s);
// The same GEMMs on the copy-wave tiles (block_m 128; H and I multiples of
// 64): four widen waves turn each stage's codes into bf16 weight tiles in
// LDS.  GEMM 2 writes bf16 pair-order rows into partial and sums them into out.
hipError_t launch_qgemm1_tiled(const QGemmArgs& a, hipStream_t s);
hipError_t launch_qgemm2_tiled(const QGemmArgs& a, hipStream_t s);

hipError_t launch_pair_gemv1(const PairGemvArgs& a, hipStream_t s);
hipError_t launch_pair_gemv2(const PairGemvArgs& a, hipStream_t s);

// Tile constants the host needs for grids and the dispatch report.
constexpr int kTiledBK = 64;
constexpr int kTiledG1Features = 128;   // act columns per GEMM 1 tile (128 gate + 128 up rows)
constexpr int kTiledG2Features = 256;   // output columns per GEMM 2 tile
constexpr int kStreamG1Features = 16;   // act columns per streaming GEMM 1 tile
constexpr int kStreamG2Features = 32;   // output columns per streaming GEMM 2 tile
constexpr int kStreamBK = 256;          // K elements per streaming LDS slice
constexpr int kPairGemvFeatures = 4;    // act columns per per-pair GEMV 1 workgroup
constexpr int kPairGemvK = 2048;        // K elements per lane-pass of the per-pair GEMVs

// Compute units of the current device (cached per device).
int device_cu_count();

// Raises a kernel's dynamic-LDS limit on the current device once; `done`
// is that kernel's own per-device flag array.  Concurrent first calls on one
// device both set the same value.
constexpr int kMaxDevices = 64;
inline hipError_t ensure_dynamic_lds(const void* kernel, int bytes, bool (&done)[kMaxDevices]) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const bool known = dev >= 0 && dev < kMaxDevices;
  if (known && done[dev]) return hipSuccess;
  err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (err == hipSuccess && known) done[dev] = true;
  return err;
}

}  // namespace moe_host
