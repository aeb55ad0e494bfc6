// fa2_api.cpp -- the C ABI declared in include/fa2.h.
//
// Validation happens here, before any HIP call, so a rejected call touches
// no device state; the launchers behind fa2_launch.hpp only ever see
// arguments that passed these checks.
#include "fa2.h"

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fa2_launch.hpp"

// Workspace of fa2_backward_noalloc: one copy per GPU, placed by the code
// object loader and held until the process ends.  Host code never passes
// this name to a kernel or a copy (on the host it is only a stand-in for the
// symbol): it uses the device address that hipGetSymbolAddress returns for
// the current device (scratch_base below).
constexpr size_t kScratchBytes = FA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_base[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up with
// hipGetSymbolAddress on the first call on that device and kept.
hipError_t scratch_base(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_base[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_base[dev] = p;
  }
  *out = g_scratch_base[dev];
  return hipSuccess;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Shared size/type checks.  Returns FA2_OK, or the status to report.
int check_sizes(int B, int H, int N, int d, int dtype) {
  if (B < 0 || H < 0 || N < 0 || d <= 0) return FA2_ERR_INVALID_ARG;
  if (dtype != FA2_F32 && dtype != FA2_BF16 && dtype != FA2_F16) return FA2_ERR_INVALID_ARG;
  if (!supported_d(d)) return FA2_ERR_UNSUPPORTED;
  // Per-head offsets are computed in int; whole-tensor offsets in size_t.
  if ((int64_t)N * d >= ((int64_t)1 << 31)) return FA2_ERR_INVALID_ARG;
  if ((int64_t)B * H >= ((int64_t)1 << 31)) return FA2_ERR_INVALID_ARG;
  return FA2_OK;
}

bool is_empty(int B, int H, int N) { return B == 0 || H == 0 || N == 0; }

// Key/value heads: 1 <= H_kv, and H_kv divides H (both may be 0 when H is).
bool valid_hkv(int H, int H_kv) { return H == 0 ? H_kv >= 0 : (H_kv >= 1 && H % H_kv == 0); }


// Decoding splits the cache over workgroups for 16-bit types at d = 128 and
// 64; other types and head sizes run the generic forward kernel, which needs
// no workspace.
bool decode_split_path(int dtype, int d) {
  return (dtype == FA2_BF16 || dtype == FA2_F16) && (d == 128 || d == 64) && !fa2::force_generic_kernels();
}

// Packed ragged batches: T rows per head, sequences of at most max_seqlen
// rows (the grid's length), device offsets cu[0..B].
int check_varlen(const int* cu, int B, int T, int max_seqlen, int d) {
  if (T < 0 || max_seqlen < 0 || max_seqlen > T) return FA2_ERR_INVALID_ARG;
  if ((int64_t)T * d >= ((int64_t)1 << 31)) return FA2_ERR_INVALID_ARG;
  if (B > 0 && !cu) return FA2_ERR_INVALID_ARG;
  if (cu && (reinterpret_cast<uintptr_t>(cu) & 3u)) return FA2_ERR_UNSUPPORTED;
  return FA2_OK;
}

// N is the sequence length (fixed) or the longest sequence (cu != null).
int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N,
                 int d, float scale, int causal, int dtype, const int* cu, int T, void* stream) {
  int st = check_sizes(B, H, N, d, dtype);
  if (st != FA2_OK) return st;
  if (!valid_hkv(H, H_kv)) return FA2_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale == 0.f) return FA2_ERR_INVALID_ARG;
  if (is_empty(B, H, N)) return FA2_OK;
  if (!q || !k || !v || !o || !lse) return FA2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA2_ERR_UNSUPPORTED;
  fa2::FwdArgs a{q, k, v, o, lse, B, H, N, d, H_kv, scale, causal != 0, dtype, static_cast<hipStream_t>(stream),
                 cu, T, 0};
  return fa2::launch_forward(a) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

// Workspace of a backward whose query side has `rows` rows and key side
// `kv_rows` ([B, H, N] and [B, H_kv, N], or [H, T] and [H_kv, T]).
size_t ws_bytes(int B, int H, int H_kv, int N, int d, int dtype, long long rows, long long kv_rows) {
  const int S = fa2::dkdv_splits(B, H_kv, H / H_kv, N, d, dtype);
  const int Sq = fa2::dq_splits(B, H, N, d, dtype);
  return fa2::ws_total_bytes((size_t)rows, d, dtype) + fa2::ws_part_bytes(kv_rows, d, S, rows, Sq);
}

// Checks of a backward call other than its workspace: FA2_OK, or the status
// to report.  *empty is set for a problem with nothing to compute.
int check_backward(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d, float scale, int dtype,
                   bool* empty) {
  *empty = false;
  int st = check_sizes(B, H, N, d, dtype);
  if (st != FA2_OK) return st;
  if (!valid_hkv(H, H_kv)) return FA2_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale == 0.f) return FA2_ERR_INVALID_ARG;
  if (is_empty(B, H, N)) {
    *empty = true;
    return FA2_OK;
  }
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA2_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, o, dO, lse, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA2_ERR_UNSUPPORTED;
  return FA2_OK;
}

// Stages stage_first .. stage_last of the backward; N as in forward_impl.
int backward_impl(int stage_first, int stage_last, const void* q, const void* k, const void* v, const void* o,
                  const void* dO, const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int N,
                  int d, float scale, int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream,
                  const int* cu = nullptr, int T = 0) {
  bool empty = false;
  const int st = check_backward(q, k, v, o, dO, lse, dq, dk, dv, B, H, H_kv, N, d, scale, dtype, &empty);
  if (st != FA2_OK || empty) return st;
  const size_t rows = cu ? (size_t)H * T : (size_t)B * H * N;
  const long long kv_rows = cu ? (long long)H_kv * T : (long long)B * H_kv * N;
  if (!workspace || workspace_bytes < ws_bytes(B, H, H_kv, N, d, dtype, (long long)rows, kv_rows))
    return FA2_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA2_ERR_UNSUPPORTED;
  float* delta = static_cast<float*>(workspace);
  float* lse2 = delta + fa2::align256(rows * sizeof(float)) / sizeof(float);
  float* part = static_cast<float*>(static_cast<void*>(static_cast<char*>(workspace) +
                                                       fa2::ws_total_bytes(rows, d, dtype)));
  const int splits = fa2::dkdv_splits(B, H_kv, H / H_kv, N, d, dtype);
  const int dq_splits = fa2::dq_splits(B, H, N, d, dtype);
  fa2::BwdArgs a{q,     k,     v,    o,    dO,     lse,       dq, dk, dv, B, H, N, d, H_kv, scale, causal != 0,
                 dtype, delta, lse2, part, splits, dq_splits, static_cast<hipStream_t>(stream), cu, T};
  for (int s = stage_first; s <= stage_last; ++s)
    if (fa2::launch_backward_stage(a, s) != hipSuccess) return FA2_ERR_LAUNCH;
  return FA2_OK;
}

}  // namespace

extern "C" {

const char* fa2_status_string(int status) {
  switch (status) {
    case FA2_OK: return "FA2_OK";
    case FA2_ERR_INVALID_ARG: return "FA2_ERR_INVALID_ARG: null pointer, negative size, bad scale or dtype, or size overflow";
    case FA2_ERR_UNSUPPORTED: return "FA2_ERR_UNSUPPORTED: head dim not in {16,32,64,128} or pointer not 16-byte aligned";
    case FA2_ERR_WORKSPACE: return "FA2_ERR_WORKSPACE: backward workspace missing or too small";
    case FA2_ERR_LAUNCH: return "FA2_ERR_LAUNCH: a HIP kernel launch failed";
    case FA2_ERR_SCRATCH:
      return "FA2_ERR_SCRATCH: the problem needs more workspace than fa2_backward_noalloc's static buffer";
    default: return "unknown fa2 status";
  }
}

int fa2_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                float scale, int causal, int dtype, void* stream) {
  return fa2_forward_ex(q, k, v, o, lse, B, H, H, N, d, scale, causal, dtype, stream);
}

int fa2_forward_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
                   int N, int d, float scale, int causal, int dtype, void* stream) {
  return forward_impl(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, dtype, nullptr, 0, stream);
}

int fa2_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens,
                       int B, int H, int H_kv, int T, int max_seqlen, int d, float scale, int causal, int dtype,
                       void* stream) {
  const int st = check_varlen(cu_seqlens, B, T, max_seqlen, d);
  if (st != FA2_OK) return st;
  return forward_impl(q, k, v, o, lse, B, H, H_kv, max_seqlen, d, scale, causal, dtype, cu_seqlens, T, stream);
}

size_t fa2_backward_workspace_size(int B, int H, int N, int d, int dtype) {
  return fa2_backward_workspace_size_ex(B, H, H, N, d, dtype);
}

size_t fa2_backward_workspace_size_ex(int B, int H, int H_kv, int N, int d, int dtype) {
  if (check_sizes(B, H, N, d, dtype) != FA2_OK || !valid_hkv(H, H_kv)) return 0;
  if (is_empty(B, H, N)) return 0;
  return ws_bytes(B, H, H_kv, N, d, dtype, (long long)B * H * N, (long long)B * H_kv * N);
}

size_t fa2_backward_workspace_size_varlen(int B, int H, int H_kv, int T, int max_seqlen, int d, int dtype) {
  if (check_sizes(B, H, max_seqlen, d, dtype) != FA2_OK || !valid_hkv(H, H_kv)) return 0;
  if (T < 0 || max_seqlen > T || (int64_t)T * d >= ((int64_t)1 << 31)) return 0;
  if (is_empty(B, H, max_seqlen)) return 0;
  return ws_bytes(B, H, H_kv, max_seqlen, d, dtype, (long long)H * T, (long long)H_kv * T);
}

int fa2_backward(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                 void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return fa2_backward_ex(q, k, v, o, dO, lse, dq, dk, dv, B, H, H, N, d, scale, causal, dtype, workspace,
                         workspace_bytes, stream);
}

int fa2_backward_ex(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                    void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d, float scale, int causal,
                    int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(1, 2, q, k, v, o, dO, lse, dq, dk, dv, B, H, H_kv, N, d, scale, causal, dtype, workspace,
                       workspace_bytes, stream);
}

int fa2_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                         const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d,
                         float scale, int causal, int dtype, void* stream) {
  bool empty = false;
  const int st = check_backward(q, k, v, o, dO, lse, dq, dk, dv, B, H, H_kv, N, d, scale, dtype, &empty);
  if (st != FA2_OK || empty) return st;
  if (fa2_backward_workspace_size_ex(B, H, H_kv, N, d, dtype) > kScratchBytes) return FA2_ERR_SCRATCH;
  void* ws = nullptr;
  if (scratch_base(&ws) != hipSuccess) return FA2_ERR_LAUNCH;
  return backward_impl(1, 2, q, k, v, o, dO, lse, dq, dk, dv, B, H, H_kv, N, d, scale, causal, dtype, ws,
                       kScratchBytes, stream);
}

int fa2_backward_varlen(const void* q, const void* k, const void* v, const void* o, const void* dO,
                        const float* lse, void* dq, void* dk, void* dv, const int* cu_seqlens, int B, int H,
                        int H_kv, int T, int max_seqlen, int d, float scale, int causal, int dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const int st = check_varlen(cu_seqlens, B, T, max_seqlen, d);
  if (st != FA2_OK) return st;
  return backward_impl(1, 2, q, k, v, o, dO, lse, dq, dk, dv, B, H, H_kv, max_seqlen, d, scale, causal, dtype,
                       workspace, workspace_bytes, stream, cu_seqlens, T);
}

int fa2_backward_stage(int stage, const void* q, const void* k, const void* v, const void* o, const void* dO,
                       const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                       int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fa2_backward_stage_ex(stage, q, k, v, o, dO, lse, dq, dk, dv, B, H, H, N, d, scale, causal, dtype,
                               workspace, workspace_bytes, stream);
}

int fa2_backward_stage_ex(int stage, const void* q, const void* k, const void* v, const void* o, const void* dO,
                          const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d,
                          float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (stage < 1 || stage > 2) return FA2_ERR_INVALID_ARG;
  return backward_impl(stage, stage, q, k, v, o, dO, lse, dq, dk, dv, B, H, H_kv, N, d, scale, causal, dtype,
                       workspace, workspace_bytes, stream);
}

int fa2_backward_stage_varlen(int stage, const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* lse, void* dq, void* dk, void* dv,
                              const int* cu_seqlens, int B, int H, int H_kv, int T, int max_seqlen, int d,
                              float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (stage < 1 || stage > 2) return FA2_ERR_INVALID_ARG;
  const int st = check_varlen(cu_seqlens, B, T, max_seqlen, d);
  if (st != FA2_OK) return st;
  return backward_impl(stage, stage, q, k, v, o, dO, lse, dq, dk, dv, B, H, H_kv, max_seqlen, d, scale, causal,
                       dtype, workspace, workspace_bytes, stream, cu_seqlens, T);
}

size_t fa2_decode_workspace_size(int B, int H, int H_kv, int N_q, int N_k, int d, int dtype) {
  if (B <= 0 || H <= 0 || N_q <= 0 || N_k <= 0 || !valid_hkv(H, H_kv)) return 0;
  if (!decode_split_path(dtype, d)) return 0;
  if ((int64_t)N_k * d >= ((int64_t)1 << 31) || (int64_t)B * H * N_q >= ((int64_t)1 << 31)) return 0;
  return fa2::decode_ws_bytes(B, H, H_kv, N_q, N_k, d);
}

int fa2_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N_q,
               int N_k, int d, float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
               void* stream) {
  if (B < 0 || H < 0 || N_q < 0 || N_k < 0 || d <= 0) return FA2_ERR_INVALID_ARG;
  if (dtype != FA2_F32 && dtype != FA2_BF16 && dtype != FA2_F16) return FA2_ERR_INVALID_ARG;
  if (!valid_hkv(H, H_kv)) return FA2_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale == 0.f) return FA2_ERR_INVALID_ARG;
  if ((int64_t)N_k * d >= ((int64_t)1 << 31) || (int64_t)N_q * d >= ((int64_t)1 << 31))
    return FA2_ERR_INVALID_ARG;
  if ((int64_t)B * H * N_q >= ((int64_t)1 << 31)) return FA2_ERR_INVALID_ARG;
  if (B == 0 || H == 0 || N_q == 0) return FA2_OK;
  if (N_k == 0 || (causal && N_q > N_k)) return FA2_ERR_INVALID_ARG;
  if (!supported_d(d)) return FA2_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || !lse) return FA2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA2_ERR_UNSUPPORTED;
  if (!decode_split_path(dtype, d)) {
    // Other types and head sizes: the generic forward kernel with the cache
    // as its keys (one workgroup per 128-query tile walks the whole cache).
    fa2::FwdArgs a{q,     k, v, o, lse, B, H, N_q, d, H_kv, scale, causal != 0, dtype, static_cast<hipStream_t>(stream),
                   nullptr, 0, N_k};
    return fa2::launch_forward(a) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
  }
  const size_t need = fa2::decode_ws_bytes(B, H, H_kv, N_q, N_k, d);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FA2_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA2_ERR_UNSUPPORTED;
  }
  fa2::DecArgs a{q,     k,           v,     o,     lse, B, H, H_kv, N_q, N_k, d, scale, causal != 0,
                 dtype, static_cast<float*>(workspace), static_cast<hipStream_t>(stream)};
  return fa2::launch_decode(a) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

}  // extern "C"
