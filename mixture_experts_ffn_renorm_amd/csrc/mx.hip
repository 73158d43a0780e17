// MXFP8 quantization of bf16 rows (the FP8 GEMM inputs: qhidden = the
// quantized copy of x, page "Mixture of Experts in vLLM - From First
// Principles to fused_moe", sub-section "The two index lists"; the MXFP8
// format named in the MLX part of the page "SGLang issue #22283" is the OCP
// microscaling one: per 32 consecutive elements one E8M0 scale 2^(c - 127)
// and 32 E4M3 bytes).
//
// A block's scale is 2^(floor(log2 amax) - 8), clamped to [2^-127, 2^127]
// (code 0 for an all-zero block); an element is v / scale rounded to the
// nearest E4M3 value with ties to the even code, saturated at 448, its sign
// kept.  Division by a power of two is exact, so the rounding decision is
// the only one and this kernel and the oracle take it on the same value.
// One thread per block: 64 bytes in, 32 bytes and one scale byte out.
#include "moe_common.h"

using namespace moe;

namespace {

// E4M3 byte of v * 2^-shared (round to nearest even, saturating, sign kept).
__device__ __forceinline__ uint32_t e4m3_of(float v, int shared) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = __builtin_ldexpf(__builtin_fabsf(v), -shared);   // exact
  uint32_t mag;
  if (!(a < 448.f)) {
    mag = 0x7Eu;                                   // 448 and above (ties at 464 go to 448)
  } else if (a < 0.015625f) {                      // below 2^-6: steps of 2^-9
    mag = (uint32_t)__builtin_rintf(a * 512.f);    // 0 .. 8 (8 is 2^-6, code 0x08)
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;        // -6 .. 8
    const float m = __builtin_ldexpf(a, -e);                         // [1, 2)
    uint32_t q = (uint32_t)__builtin_rintf((m - 1.f) * 8.f);         // exact operands
    if (q == 8u) { q = 0u; ++e; }
    mag = ((uint32_t)(e + 7) << 3) | q;
  }
  return sign | mag;
}

__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ src,
                                                          long long nblocks, int K,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
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
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);   // 0: zero or subnormal
  int shared = ef == 0 ? -127 : ef - 127 - 8;
  shared = shared < -127 ? -127 : (shared > 127 ? 127 : shared);
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

}  // namespace

namespace moe_host {

hipError_t launch_mx_quantize(const uint16_t* src, int rows, int K, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  const long long nblocks = (long long)rows * (K / 32);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s,
                     src, nblocks, K, codes, scales);
  return hipGetLastError();
}

}  // namespace moe_host
