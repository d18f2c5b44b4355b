// calibrate.hip -- a plain streaming copy, the measured HBM reference for the
// memory-bound kernels (the decode step reads and writes its state once per
// token).  Each thread moves 16-byte pieces; a grid-stride loop keeps four
// independent loads in flight per thread before their stores.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/mamba_mi355x.h"

namespace {

__global__ __launch_bounds__(256) void stream_copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                                          uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const float4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// One pass, each workgroup over a contiguous run of 4 x 256 pieces (four loads in
// flight per thread); NT: non-temporal loads and stores.
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ __launch_bounds__(256) void block_copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                         uint64_t n) {
  const uint64_t base = (uint64_t)blockIdx.x * 1024 + threadIdx.x;
  f32x4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t i = base + 256 * k;
    if (i < n) v[k] = NT ? __builtin_nontemporal_load(src + i) : src[i];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t i = base + 256 * k;
    if (i < n) {
      if (NT) __builtin_nontemporal_store(v[k], dst + i);
      else dst[i] = v[k];
    }
  }
}

// In place: each piece read and written back (the decode step's access to its state).
template <bool NT>
__global__ __launch_bounds__(256) void inplace_kernel(f32x4* p, uint64_t n) {
  const uint64_t base = (uint64_t)blockIdx.x * 1024 + threadIdx.x;
  f32x4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t i = base + 256 * k;
    if (i < n) v[k] = NT ? __builtin_nontemporal_load(p + i) : p[i];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t i = base + 256 * k;
    if (i < n) {
      if (NT) __builtin_nontemporal_store(v[k], p + i);
      else p[i] = v[k];
    }
  }
}

}  // namespace

extern "C" int mamba_calibrate_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (bytes == 0) return MAMBA_OK;
  if (!src || !dst) return MAMBA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | bytes) & 15u) return MAMBA_ERR_ALIGN;
  const uint64_t n = bytes / 16;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const auto s4 = static_cast<const float4*>(src);
  const auto d4 = static_cast<float4*>(dst);
  if (blocks > 0) {
    if (blocks > (1 << 20)) return MAMBA_ERR_DIM;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, s4, d4, n);
  } else {
    const uint64_t nb = (n + 1023) / 1024;
    if (blocks < -3 || nb > 0xffffffffull) return MAMBA_ERR_DIM;
    const auto sv = static_cast<const f32x4*>(src);
    const auto dv = static_cast<f32x4*>(dst);
    if (blocks == 0) hipLaunchKernelGGL(block_copy_kernel<false>, dim3((unsigned)nb), dim3(256), 0, st, sv, dv, n);
    else if (blocks == -1) hipLaunchKernelGGL(block_copy_kernel<true>, dim3((unsigned)nb), dim3(256), 0, st, sv, dv, n);
    else if (blocks == -2) hipLaunchKernelGGL(inplace_kernel<false>, dim3((unsigned)nb), dim3(256), 0, st, dv, n);
    else hipLaunchKernelGGL(inplace_kernel<true>, dim3((unsigned)nb), dim3(256), 0, st, dv, n);
  }
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}
