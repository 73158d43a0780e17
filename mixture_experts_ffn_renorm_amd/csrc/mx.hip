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
// One thread per block: 64 bytes in, 32 bytes and one scale byte out (the
// block quantizer and the E4M3 rounding are in moe_common.h).
#include "moe_common.h"

using namespace moe;

namespace {

__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ src,
                                                          long long nblocks, int K,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  mx_quantize_block(src, K, b, codes, scales);
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
