// fa2_launch.hpp -- internal interface between the C ABI (fa2_api.cpp) and the
// kernel launchers.  Arguments arrive here already validated: sizes are
// positive, d is one of 16/32/64/128, pointers are non-null and 16-byte
// aligned, and the workspace is large enough.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdlib.h>

namespace fa2 {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kF16 = 2;

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
  // Packed ragged batch: device sequence offsets [B + 1] (null: fixed length
  // N, layout [B, H, N, d]); with them the layout is [H, T, d] and N is the
  // longest sequence.
  const int* cu;
  int T;
  // Decoding through the generic kernel: k, v hold Nk rows per key/value
  // head ([B, Hkv, Nk, d]) and the N queries are their last positions (0: the
  // keys are the query rows).
  int Nk;
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
  float* part;   // splits > 1: fp32 partial dK then dV, [splits][B, Hkv, N, d] each;
                 // dq_splits > 1: fp32 partial dQ, [dq_splits][B, H, N, d] (stage 1,
                 // before stage 2 reuses the area)
  int splits;    // workgroups that share one key tile (its query heads, or fp32: its query tiles)
  int dq_splits; // fp32: workgroups that share one query tile's walk over the key tiles
  hipStream_t stream;
  const int* cu;  // as FwdArgs
  int T;
};

// Workspace layout: D = rowsum(dO * O), then LSE * log2(e), each float
// [B, H, N] padded to 256 B (written by the dQ kernel of stage 1); then, when
// the dK/dV stage splits a key tile's work over several workgroups, their
// fp32 partial dK and dV.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t ws_total_bytes(size_t rows, int /*d*/, int /*dtype*/) { return 2 * align256(rows * sizeof(float)); }

// How many workgroups share one key/value head's group of G query heads in
// the dK/dV stage.  One workgroup per (key/value head, 128-key tile) walks
// the whole group, which leaves few workgroups when G is large; the 16-bit,
// d = 128 kernel then splits the group over S workgroups (S divides G) until
// there are at least 1024 of them (four per CU: with causal masking the key
// tiles differ in cost, and two per CU left the heavy ones as a tail), and a
// second kernel sums the S partial results in a fixed order.
//
// fp32 runs the generic dK/dV kernel at one workgroup per CU.  There the
// split is over query tiles instead: when the key tiles leave fewer than
// 512 workgroups, each key tile's walk over the query tiles is cut into S
// consecutive pieces (as long as the longest walk keeps at least 4 query
// tiles per piece), and the same second kernel sums the pieces' partials.
// With causal masking this also shortens the heaviest workgroup's walk.
//
// At d <= 64 a small fp32 grid first halves the walks inside each workgroup
// (fp32_paired_walks): the dK/dV workgroup covers 64 keys and its two waves
// per key group take alternate query steps, the dQ workgroup covers 64 rows
// and its two waves per row group take alternate key tiles, each pair adding
// its accumulators in LDS at the end.  That doubles the grid with no partial
// sums in memory; the S pieces above are then cut from what is left.  (A
// walk of fewer than 256 keys or queries has too few steps to share.)
inline bool fp32_paired_walks(int B, int heads, int N, int d, int dtype) {
  return dtype == kF32 && d <= 64 && N >= 256 && (long long)((N + 127) / 128) * B * heads < 512;
}
inline int dkdv_splits(int B, int Hkv, int G, int N, int d, int dtype) {
  if (dtype == kF32) {
    const int br = d >= 64 ? 32 : 64;  // query rows per step of the fp32 generic kernel
    const int steps = (N + br - 1) / br;
    const bool paired = fp32_paired_walks(B, Hkv, N, d, dtype);
    const int bc = paired ? 64 : 128;    // keys per workgroup
    const int per = paired ? 8 : 4;      // query steps a piece keeps at least
    const long long base = (long long)((N + bc - 1) / bc) * B * Hkv;
    int S = 1;
    while (base * S < 512 && steps / (S + 1) >= per) ++S;
    return S;
  }
  if (G <= 1 || d != 128) return 1;
  const long long base = (long long)((N + 127) / 128) * B * Hkv;
  int S = 1;
  while (S < G && base * S < 1024) {
    ++S;
    while (G % S) ++S;
  }
  return S;
}
// The same split on the dQ side (fp32, generic kernel at one workgroup per
// CU): with fewer than 512 query-tile workgroups, each query tile's walk
// over the 32-key tiles is cut into S pieces while the longest walk keeps at
// least 8 key tiles per piece (shorter walks do not pay for the second
// launch); a second kernel sums the fp32 partial dQ.
inline int dq_splits(int B, int H, int N, int d, int dtype) {
  if (dtype != kF32) return 1;
  const int steps = (N + 31) / 32;
  const bool paired = fp32_paired_walks(B, H, N, d, dtype);
  const int br = paired ? 64 : 128;    // query rows per workgroup
  const int per = paired ? 16 : 8;     // key tiles a piece keeps at least
  const long long base = (long long)((N + br - 1) / br) * B * H;
  int S = 1;
  while (base * S < 512 && steps / (S + 1) >= per) ++S;
  return S;
}
// kv_rows: rows of dK ([B, Hkv, N] or, packed, [Hkv, T]); rows: rows of dQ.
// Stage 1's partial dQ and stage 2's partial dK, dV share one area.
inline size_t ws_part_bytes(long long kv_rows, int d, int S, long long rows = 0, int Sq = 1) {
  const size_t kv = S > 1 ? 2 * align256((size_t)S * kv_rows * d * sizeof(float)) : 0;
  const size_t q = Sq > 1 ? align256((size_t)Sq * rows * d * sizeof(float)) : 0;
  return kv > q ? kv : q;
}

// Decoding (bf16 or fp16, d = 128): N_q queries [B, H, N_q, d] against a cache
// k, v [B, Hkv, N_k, d]; the workspace holds the chunks' partial results.
struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, Nq, Nk, d;
  float scale;
  bool causal;
  int dtype;
  float* workspace;
  hipStream_t stream;
};

// How the decode pass is cut: row blocks of 32 of the G * N_q rows of a
// key/value head, and the cache split into chunks of chunk_blocks 32-key
// blocks.  Splits are added until there are about kDecodeWorkgroups
// workgroups (one wave each, two per CU: one round over the device; more,
// shorter chunks measured slower, each chunk paying its own load latency
// before its ring fills), keeping chunks of at least 4 blocks; no chunk is
// left empty.
constexpr long long kDecodeWorkgroups = 512;
struct DecodePlan {
  int row_blocks, splits, chunk_blocks;
};
inline DecodePlan decode_plan(int B, int H, int Hkv, int Nq, int Nk) {
  DecodePlan p;
  const long long M = (long long)(H / Hkv) * Nq;
  p.row_blocks = (int)((M + 31) / 32);
  const int nbk = (Nk + 31) / 32;
  const long long base = (long long)B * Hkv * p.row_blocks;
  long long want = (kDecodeWorkgroups + base - 1) / base;
  const long long most = nbk / 4 > 1 ? nbk / 4 : 1;
  if (want > most) want = most;
  if (want < 1) want = 1;
  p.chunk_blocks = (int)((nbk + want - 1) / want);
  p.splits = (nbk + p.chunk_blocks - 1) / p.chunk_blocks;
  return p;
}
inline size_t decode_ws_bytes(int B, int H, int Hkv, int Nq, int Nk, int d) {
  const DecodePlan p = decode_plan(B, H, Hkv, Nq, Nk);
  if (p.splits <= 1) return 0;
  const size_t rows = (size_t)B * H * Nq;
  return align256((size_t)p.splits * rows * d * sizeof(float)) + align256((size_t)p.splits * rows * sizeof(float));
}

// FA2_FORCE_GENERIC set to anything but "0" in the environment makes every
// call take the generic kernels (register-staged tiles) instead of the tuned
// 16-bit d = 128 and d = 64 ones, and decoding the unsplit path: a second,
// independent tiling of the same arithmetic, for checking the two against
// each other.  Read on the host at every call; no state is kept.
inline bool force_generic_kernels() {
  const char* e = getenv("FA2_FORCE_GENERIC");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

hipError_t launch_forward(const FwdArgs& a);
hipError_t launch_decode(const DecArgs& a);
// stage 1: the dQ kernel, which also writes D = rowsum(dO * O) and
// LSE * log2(e) to the workspace; 2: the dK/dV kernel.
hipError_t launch_backward_stage(const BwdArgs& a, int stage);

}  // namespace fa2
