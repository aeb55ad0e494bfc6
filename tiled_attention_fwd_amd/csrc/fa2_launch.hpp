// fa2_launch.hpp -- internal interface between the C ABI (fa2_api.cpp) and the
// kernel launchers.  Arguments arrive here already validated: sizes are
// positive, d is one of 16/32/64/128, pointers are non-null and 16-byte
// aligned, and the workspace is large enough.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa2 {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;
  bool causal;
  int dtype;
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, H, N, d;
  float scale;
  bool causal;
  int dtype;
  float* delta;  // [B, H, N] inside the workspace
  float* dq_acc;  // [B, H, N, d] fp32 accumulator (dq itself in fp32 mode)
  hipStream_t stream;
};

// Workspace layout: delta first, then (bf16 mode) the fp32 dQ accumulator,
// each section starting on a 256-byte boundary.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t ws_delta_bytes(size_t rows) { return align256(rows * sizeof(float)); }
inline size_t ws_total_bytes(size_t rows, int d, int dtype) {
  return ws_delta_bytes(rows) + (dtype == kBF16 ? align256(rows * (size_t)d * sizeof(float)) : 0);
}

hipError_t launch_forward(const FwdArgs& a);
// stage 1: D and accumulator zeroing; 2: the key-tile kernel; 3: dQ to bf16.
hipError_t launch_backward_stage(const BwdArgs& a, int stage);

}  // namespace fa2
