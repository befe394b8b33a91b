// moe_pack.hip -- weight preparation: MXFP4 E8M0 scale bytes from the row
// grid of the OCP MX definition ([rows][k/32], one byte per 32 elements)
// into the tiled layout the layer reads, in which the scales of 16
// consecutive rows for one K-block of 256 elements are one 128-byte line:
// byte j of row n's K-block kb goes to ((n/16)*(k/256) + kb)*128 + (n%16)*8 + j.
// A 16-row weight tile's scale load then touches one line instead of 16.
#include "moe.h"
#include "moe_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kPackThreads = 256;

// One thread per (row, K-block): 8 scale bytes moved as one 64-bit word
// (a row's K-block starts at a multiple of 8 bytes since k/32 is).
__global__ __launch_bounds__(kPackThreads) void pack_mxfp4_scales(const uint64_t* __restrict__ src,
                                                                   uint64_t* __restrict__ dst, size_t rows,
                                                                   size_t kb) {
  const size_t t = (size_t)blockIdx.x * kPackThreads + threadIdx.x;
  if (t >= rows * kb) return;
  const size_t n = t / kb, b = t - n * kb;
  dst[((n >> 4) * kb + b) * 16 + (n & 15)] = src[t];
}

}  // namespace

extern "C" int moe_pack_mxfp4_scales(const uint8_t* src, uint8_t* dst, int rows, int k, void* stream) {
  if (!src || !dst) return MOE_ERR_NULL;
  if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return MOE_ERR_ALIGN;
  if (rows <= 0 || rows % 16 || k <= 0 || k % 256) return MOE_ERR_SHAPE;
  const size_t kb = (size_t)k / 256, bytes = (size_t)rows * kb * 8;
  if (src < dst + bytes && dst < src + bytes) return MOE_ERR_ALIAS;
  const size_t n = (size_t)rows * kb;
  const unsigned blocks = (unsigned)((n + kPackThreads - 1) / kPackThreads);
  hipLaunchKernelGGL(pack_mxfp4_scales, dim3(blocks), dim3(kPackThreads), 0, (hipStream_t)stream,
                     (const uint64_t*)src, (uint64_t*)dst, (size_t)rows, kb);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return MOE_OK;
  moe::set_last_hip((int)e);
  return MOE_ERR_HIP;
}
