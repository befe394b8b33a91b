// moe_probe.hip -- measurement helper: a plain streaming read of device
// memory, to put the layer's achieved HBM bandwidth beside what this GPU
// streams for pure reads (the published 8 TB/s is the datasheet figure).
//
// Each thread reads 16-byte words with a grid stride, eight loads in flight
// per iteration, and folds them into an xor that one thread per workgroup
// stores to sink[blockIdx.x], so no load can be dropped.  The buffer is read
// exactly once per launch.
#include "moe.h"
#include "moe_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void stream_read(const u32x4* __restrict__ buf, size_t n16,
                                                             uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) v[j] = __builtin_nontemporal_load(buf + i + j * stride);
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) acc ^= v[j];
  }
  for (; i < n16; i += stride) acc ^= buf[i];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
  __shared__ uint32_t part[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) s ^= part[w];
    sink[blockIdx.x] = s;
  }
}

}  // namespace

extern "C" int moe_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!buf || !sink) return MOE_ERR_NULL;
  if (((uintptr_t)buf & 15u) || (bytes & 15u)) return MOE_ERR_ALIGN;
  if (blocks < 1 || blocks > (1 << 20)) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(kProbeThreads), 0, (hipStream_t)stream,
                     (const u32x4*)buf, bytes / 16, sink);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return MOE_OK;
  moe::set_last_hip((int)e);
  return MOE_ERR_HIP;
}
