// s6_internal.h -- host-side plan and launcher declarations shared by the
// C-ABI layer (api.cpp) and the kernel translation units.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace s6 {

enum IoType { kIoF32 = 0, kIoBF16 = 1 };

// Arguments of one forward scan; pointers are device pointers.
struct ScanArgs {
  const void* u;
  const void* delta;
  const float* bias;   // may be null
  const float* A;
  const void* B;
  const void* C;
  const float* dskip;  // may be null
  const void* z;       // may be null
  const float* h0;     // may be null
  void* out;
  float* last;         // may be null
  float* agg_h;        // workspace: (batch, nchunks, D, N) chunk states / carries
  float* agg_s;        // workspace: (batch, nchunks, D) chunk sums of dt
  int64_t batch, L, D;
  int64_t chunk_len;
  int32_t nchunks;
  int32_t softplus;
};

struct StepArgs {
  float* state;
  const void* u;
  const void* delta;
  const float* bias;
  const float* A;
  const void* B;
  const void* C;
  const float* dskip;
  const void* z;
  void* out;
  int64_t batch, D;
  int32_t softplus;
};

// Execution plan of a forward scan, a pure function of the shape.
struct ScanPlan {
  int32_t nchunks;    // L is cut into this many chunks of chunk_len tokens
  int64_t chunk_len;
  int32_t block;      // threads per workgroup (64 channels per wave)
  size_t ws_bytes;    // workspace the plan needs (0 when nchunks == 1)
};

ScanPlan plan_scan(int64_t batch, int64_t L, int64_t D, int64_t N);

bool dstate_supported(int64_t N);

// Enqueue the kernels of one scan / one decode step on `stream`.
hipError_t launch_scan(const ScanArgs& a, const ScanPlan& p, int io, int N, hipStream_t stream);
hipError_t launch_step(const StepArgs& a, int io, int N, hipStream_t stream);

}  // namespace s6
