// fa2_swz.hpp -- swizzled LDS tiles and direct global-to-LDS loads (gfx950).
//
// Shared by the forward, backward and decode kernels for the 16-bit types at
// d = 128, whose tiles are stored unpadded, 256 bytes per row, and by the
// d = 64 dK/dV kernel (128-byte rows, swz64); all are filled by direct loads
// (no register staging).
#pragma once
#include "fa2_common.hpp"

namespace fa2 {
namespace tiles {

template <int V>
struct IntC {
  static constexpr int value = V;
};

// Tiles are stored unpadded, 256 bytes per row, with the sixteen 16-byte
// chunks of row r permuted as chunk ^ swz(r).  swz is a permutation over any
// 16 consecutive rows, so the 16 lanes that read one chunk of 16 rows hit
// all 64 banks once; and rows r..r+3 (r % 4 == 0) move a 64-byte column
// block to four different 64-byte positions, so a transposed read, whose 32
// lanes take one column block from 4 rows, also covers every bank once.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

typedef __attribute__((address_space(3))) void lds_void;

// Direct global-to-LDS loads.  They are issued from inline assembly so that
// the compiler does not see them as LDS writes: it would otherwise make the
// first LDS read after each one wait for it, whatever buffer it reads.  The
// kernels therefore order them by hand: wait_vmem() and a barrier before any
// read of the data they bring.
// M0 is named as clobbered; clang notes that it is a reserved register, which
// is what is wanted here (nothing keeps a value in M0 across these).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ unsigned lds_off(const void* p) { return (unsigned)(size_t)(const lds_void*)p; }
// 16 bytes per lane from 64-bit global address g into LDS at lds + 16*lane
// (lds wave-uniform).
__device__ __forceinline__ void dload16(const void* g, const void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_off(lds)) : "memory", "m0");
}
// 4 bytes per lane into LDS at lds + 4*lane.
__device__ __forceinline__ void dload4(const void* g, const void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_off(lds)) : "memory", "m0");
}
// Raw buffer resource over `bytes` bytes at `base` (stride 0, gfx9 data
// format 32); base must be wave-uniform.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, unsigned bytes) {
  const size_t a = (size_t)base;
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((unsigned)a);
  r.y = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000u;
  return r;
}
// 16 bytes per lane from buffer offset voffset + soffset into LDS at
// lds + 16*lane (soffset and lds wave-uniform).
__device__ __forceinline__ void bload16(u32x4 r, int voffset, int soffset, const void* lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voffset), "s"(r),
               "s"(lds_off(lds)), "s"(soffset)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt at their maxima) through the builtin,
// so that the compiler's own wait tracking sees it.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(4): all but the last four vector memory operations done.
__device__ __forceinline__ void wait_vmem4() { __builtin_amdgcn_s_waitcnt(0x0F74); }
// s_waitcnt vmcnt(n): all but the last n vector memory operations done.
template <int n>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(n >= 0 && n < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | n);
}

// Byte offsets inside a swizzled tile.  The swizzle only touches bits 4..7
// of a row's byte offset, so every fragment offset a lane needs is one of a
// few per-lane values XORed with a compile-time constant.
//   Row fragment (lane row l32, chunk 2c + h):  rofs ^ (c << 5)
//   Transpose fragment (t, column block b), the two 4-row halves:
//     t*4096 + tofs0 + ((b ^ kk) << 6)  and  t*4096 + tofs1 + ((b ^ kk) << 6)
struct SwzOffsets {
  int rofs, tofs0, tofs1, kk;
};
__device__ __forceinline__ SwzOffsets swz_offsets(int lane) {
  const int l32 = lane & 31, h = lane >> 5, j = lane & 15;
  SwzOffsets o;
  o.rofs = l32 * 256 + ((h ^ swz(l32)) << 4);
  const int r0 = 4 * h + (j >> 2);  // < 8, so swz(r0 + 8) = swz(r0) ^ 2
  const int s0 = swz(r0);
  const int c1 = 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
  o.tofs0 = r0 * 256 + ((c1 ^ (s0 & 3)) << 4) + 8 * (j & 1);
  o.tofs1 = (r0 + 8) * 256 + ((c1 ^ ((s0 & 3) ^ 2)) << 4) + 8 * (j & 1);
  o.kk = s0 >> 2;
  return o;
}
// 128-byte rows (d = 64): chunk c (0..7) of row r is stored at c ^ swz64(r).
// Over 16 consecutive rows the 8 even rows take 8 distinct values, and so do
// the 8 odd ones, so 16 lanes reading one chunk of 16 rows hit every bank
// once; bit 2 is (r >> 1) & 1, so rows r and r + 2 of a transposed read's
// 4-row group sit in different 64-byte halves and its 32 lanes also cover
// every bank once.
__device__ __forceinline__ int swz64(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
// Lane offsets for 128-byte rows, as swz_offsets: row fragment (chunk
// 2c + h of row l32) at rofs ^ (c << 5); transpose fragment (t, column
// block b) at t*2048 + tofs{0,1} + ((b ^ kk) << 6).
__device__ __forceinline__ SwzOffsets swz_offsets64(int lane) {
  const int l32 = lane & 31, h = lane >> 5, j = lane & 15;
  SwzOffsets o;
  o.rofs = l32 * 128 + ((h ^ swz64(l32)) << 4);
  const int r0 = 4 * h + (j >> 2);  // < 8: swz64(r0 + 8) = swz64(r0) ^ 2
  const int f0 = (r0 >> 2) & 3;
  const int c1 = 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
  o.tofs0 = r0 * 128 + ((c1 ^ f0) << 4) + 8 * (j & 1);
  o.tofs1 = (r0 + 8) * 128 + ((c1 ^ (f0 ^ 2)) << 4) + 8 * (j & 1);
  o.kk = (r0 >> 1) & 1;
  return o;
}
__device__ __forceinline__ u32x4 lds16(const void* base, int byte_off) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + byte_off);
}
// Transposed fragment (see load_rowcontract) from two byte offsets.
__device__ __forceinline__ u32x4 tr_frag(const void* base, int off0, int off1) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const char* b = reinterpret_cast<const char*>(base);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + off0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + off1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
}  // namespace tiles
}  // namespace fa2
