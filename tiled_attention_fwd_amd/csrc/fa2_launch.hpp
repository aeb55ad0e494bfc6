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
  float* part;   // splits > 1: fp32 partial dK then dV, [splits][B, Hkv, N, d] each
  int splits;    // workgroups that share one key/value head's query-head group
  hipStream_t stream;
};

// Workspace layout: D = rowsum(dO * O), then LSE * log2(e), each float
// [B, H, N] padded to 256 B; then, when a grouped-query backward splits each
// group over several workgroups, their fp32 partial dK and dV.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t ws_total_bytes(size_t rows, int /*d*/, int /*dtype*/) { return 2 * align256(rows * sizeof(float)); }

// How many workgroups share one key/value head's group of G query heads in
// the dK/dV stage.  One workgroup per (key/value head, 128-key tile) walks
// the whole group, which leaves few workgroups when G is large; the bf16,
// d = 128 kernel then splits the group over S workgroups (S divides G) until
// there are at least 1024 of them (four per CU: with causal masking the key
// tiles differ in cost, and two per CU left the heavy ones as a tail), and a
// second kernel sums the S partial results in a fixed order.
inline int dkdv_splits(int B, int Hkv, int G, int N, int d, int dtype) {
  if (G <= 1 || d != 128 || dtype != kBF16) return 1;
  const long long base = (long long)((N + 127) / 128) * B * Hkv;
  int S = 1;
  while (S < G && base * S < 1024) {
    ++S;
    while (G % S) ++S;
  }
  return S;
}
inline size_t ws_part_bytes(int B, int Hkv, int N, int d, int S) {
  return S > 1 ? 2 * align256((size_t)S * B * Hkv * N * d * sizeof(float)) : 0;
}

hipError_t launch_forward(const FwdArgs& a);
// stage 1: D = rowsum(dO * O); 2: the dK/dV kernel; 3: the dQ kernel.
hipError_t launch_backward_stage(const BwdArgs& a, int stage);

}  // namespace fa2
