// bf16 -> fp16 copy of the attention inputs (the operand format of the fp16
// attention kernels). Elementwise and bound by HBM: each thread moves 16-byte
// chunks (eight values) with a grid-stride loop.
#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// Two bf16 values (one 32-bit word) -> two fp16 values; `bad` is set when a
// biased exponent reaches 127 + 16 (|x| >= 65536, inf or NaN).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, bool& bad) {
  const uint32_t e0 = (w >> 7) & 0xffu, e1 = (w >> 23) & 0xffu;
  bad |= (e0 >= 143u) | (e1 >= 143u);
  const float f0 = __builtin_bit_cast(float, w << 16), f1 = __builtin_bit_cast(float, w & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{f0, f1}, f16x2));
}

__global__ void __launch_bounds__(256) convert_f16_kernel(const u32x4* src, u32x4* dst, int64_t chunks,
                                                          int32_t* status) {
  bool bad = false;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += stride) {
    const u32x4 w = src[c];
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = bf16x2_to_f16x2(w[j], bad);
    dst[c] = r;
  }
  if (bad) *status = VS_ERR_RANGE;   // every writer stores the same value
}

int launch_convert_f16(const void* src, void* dst, int64_t n, int32_t* status, hipStream_t stream) {
  const int64_t chunks = n / 8;
  const int tpb = 256;
  int64_t blocks = (chunks + tpb - 1) / tpb;
  if (blocks > 8192) blocks = 8192;   // 32 workgroups per CU, then stride
  hipLaunchKernelGGL(convert_f16_kernel, dim3((unsigned)blocks), dim3(tpb), 0, stream, (const u32x4*)src,
                     (u32x4*)dst, chunks, status);
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

}  // namespace vs
