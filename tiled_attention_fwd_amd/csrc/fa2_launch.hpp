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
  int Hkv;  // key/value heads (divides H; H / Hkv query heads share one)
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
  int Hkv;  // key/value heads (divides H; H / Hkv query heads share one)
  float scale;
  bool causal;
  int dtype;
  float* delta;  // D = rowsum(dO * O), [B, H, N] inside the workspace
  float* lse2;   // LSE * log2(e), [B, H, N] inside the workspace
  hipStream_t stream;
};

// Workspace layout: D = rowsum(dO * O), then LSE * log2(e), each float
// [B, H, N] padded to 256 B.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t ws_total_bytes(size_t rows, int /*d*/, int /*dtype*/) { return 2 * align256(rows * sizeof(float)); }

hipError_t launch_forward(const FwdArgs& a);
// stage 1: D = rowsum(dO * O); 2: the dK/dV kernel; 3: the dQ kernel.
hipError_t launch_backward_stage(const BwdArgs& a, int stage);

}  // namespace fa2
