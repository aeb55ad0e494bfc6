// fa2_common.hpp -- gfx950 building blocks shared by the attention kernels.
//
// Everything here is about mapping tiles onto the CDNA4 32x32 MFMA:
//   * bf16 operands use v_mfma_f32_32x32x16_bf16 (8 bf16 per lane per operand),
//   * fp32 operands use v_mfma_f32_32x32x2_f32 (1 float per lane per operand),
// both accumulating a 32x32 fp32 block held as 16 floats per lane.
//
// Lane conventions of a wave64 (l = lane, l32 = l % 32, h = l / 32):
//   A operand  (M x K): lane supplies row  m = l32, contraction slots of half h
//   B operand  (K x N): lane supplies column n = l32, contraction slots of half h
//   accumulator (M x N): lane holds column n = l32 and rows
//                        acc_row(r, h) = 8*(r/4) + 4*h + r%4 for r = 0..15.
// A product only needs A and B to number their contraction slots the same
// way, so every operand here is fetched as one 16-byte fragment per lane
// ("chunk"): CH = 16 / sizeof(element) consecutive contraction elements.
// For bf16 a chunk is one MFMA (half h covers elements 8h..8h+7 of a
// 16-wide step); for fp32 it is four MFMAs (element e of the fragment
// feeds step e).
//
// When the second product of an attention step contracts over the ROW
// index of a previous accumulator (P or dS), the lane already holds the
// right column and only needs its 16 accumulator values packed into chunks.
// The matching A operand is read from an LDS tile stored transposed, with
// the contraction index x at position swap_bits23(x) inside each group of
// 16, which makes the rows a lane needs for one chunk contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Reinterpret whole 16-byte fragments.  (Bit-casting a single element of an
// ext_vector, as in __builtin_bit_cast(float, v[e]), is miscompiled by the
// ROCm 7.2 clang inside unrolled loops -- every iteration reads element 0 --
// so elements are only ever taken from vectors of the wanted type.)
__device__ __forceinline__ f32x4 as_f32x4(u32x4 v) { return __builtin_bit_cast(f32x4, v); }
__device__ __forceinline__ u32x4 as_u32x4(f32x4 v) { return __builtin_bit_cast(u32x4, v); }

// Compile-time bool carried by a value (selects masked / unmasked code paths).
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Lazy rescaling of the online softmax: the running max (base-2 units) only
// moves when a block's max exceeds it by more than this, so weights stay
// below 2^kSlack, harmless in fp32 accumulators and bf16 operands.
constexpr float kSlack = 8.0f;

template <typename T>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int CH = 4;  // elements per 16-byte fragment
};
template <>
struct Elt<__bf16> {
  static constexpr int CH = 8;
};
template <>
struct Elt<_Float16> {
  static constexpr int CH = 8;
};

__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Position of contraction index x inside a transposed LDS tile.
__device__ __forceinline__ int swap_bits23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// First LDS position of chunk t (accumulator registers CH*t .. CH*t+CH-1) of
// a 32-row accumulator block, for lane half h, in a swap_bits23 tile.
template <int CH>
__device__ __forceinline__ int chunk_pos(int t, int h) {
  const int r0 = CH * t;
  return 16 * (r0 >> 3) + 8 * h + 4 * ((r0 >> 2) & 1);
}

// acc += A_fragment * B_fragment over one 16-byte chunk of the contraction.
template <typename T>
__device__ __forceinline__ void mfma_chunk(f32x16& acc, u32x4 a, u32x4 b);

template <>
__device__ __forceinline__ void mfma_chunk<__bf16>(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_chunk<_Float16>(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0,
                                                0, 0);
}

template <>
__device__ __forceinline__ void mfma_chunk<float>(f32x16& acc, u32x4 a, u32x4 b) {
  const f32x4 af = as_f32x4(a), bf = as_f32x4(b);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], bf[e], acc, 0, 0, 0);
}

// A negative scale: scale * q.k = |scale| * (-q).k.  The kernels that keep
// a running maximum of raw scores (forward, decoding) scale that maximum by
// the factor, which is only the maximum of the scaled scores for a factor
// >= 0; so with a negative factor they flip the sign bits of their query
// fragments once (exact in every type) and work with |factor|.
template <typename T>
__device__ __forceinline__ void negate_fragments_if(u32x4* f, int n, float& sl2) {
  if (sl2 < 0.f) {
    constexpr unsigned kSign = sizeof(T) == 4 ? 0x80000000u : 0x80008000u;
#pragma unroll
    for (int c = 0; c < n; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) f[c][e] ^= kSign;
    sl2 = -sl2;
  }
}

// Pack accumulator registers CH*t .. CH*t+CH-1 into one B-operand fragment
// (bf16, fp16: round to nearest even, two per dword).
template <typename T>
__device__ __forceinline__ u32x4 pack_chunk(const f32x16& x, int t);

template <>
__device__ __forceinline__ u32x4 pack_chunk<__bf16>(const f32x16& x, int t) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f32x2 pr = {x[8 * t + 2 * w], x[8 * t + 2 * w + 1]};
    r[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
  }
  return r;
}

template <>
__device__ __forceinline__ u32x4 pack_chunk<_Float16>(const f32x16& x, int t) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f32x2 pr = {x[8 * t + 2 * w], x[8 * t + 2 * w + 1]};
    r[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, f16x2));
  }
  return r;
}

template <>
__device__ __forceinline__ u32x4 pack_chunk<float>(const f32x16& x, int t) {
  return as_u32x4(f32x4{x[4 * t], x[4 * t + 1], x[4 * t + 2], x[4 * t + 3]});
}

// acc + sum of the CH values of a packed fragment (bf16: v_dot2 with ones,
// i.e. the sum of exactly the rounded weights the MFMA consumes).
template <typename T>
__device__ __forceinline__ float add_fragment_sum(float acc, u32x4 v);

template <>
__device__ __forceinline__ float add_fragment_sum<__bf16>(float acc, u32x4 v) {
  const bf16x8 b = __builtin_bit_cast(bf16x8, v);
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 6, 7), one, acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float add_fragment_sum<_Float16>(float acc, u32x4 v) {
  const f16x8 b = __builtin_bit_cast(f16x8, v);
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(b, b, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(b, b, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(b, b, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(b, b, 6, 7), one, acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float add_fragment_sum<float>(float acc, u32x4 v) {
  const f32x4 f = as_f32x4(v);
  return acc + ((f[0] + f[1]) + (f[2] + f[3]));
}

// Store 4 consecutive fp32 values as 4 elements of T (8 or 16 bytes).
template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
}

template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* dst, float a, float b, float c, float d) {
  f32x2 lo = {a, b}, hi = {c, d};
  *reinterpret_cast<u32x2*>(dst) = u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                                         __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2))};
}

template <>
__device__ __forceinline__ void store4<_Float16>(_Float16* dst, float a, float b, float c, float d) {
  f32x2 lo = {a, b}, hi = {c, d};
  *reinterpret_cast<u32x2*>(dst) = u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, f16x2)),
                                         __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, f16x2))};
}

// A single element converted from fp32.
template <typename T>
__device__ __forceinline__ T from_f32(float x) {
  return static_cast<T>(x);
}

// Transposed write of a 4-row x CH-column block held as four 16-byte row
// fragments: for every column x, the 4 values (rows 0..3) are written as one
// contiguous group at dst_col(x).  `row_stride` is the LDS tile row length
// in elements; `col0` is the first destination row of the transposed tile
// and `pos` the destination position of row 0 (rows 1..3 follow it).
template <typename T>
__device__ __forceinline__ void write_transposed4(T* tile, int row_stride, int col0, int pos,
                                                  const u32x4 (&r)[4]);

template <>
__device__ __forceinline__ void write_transposed4<float>(float* tile, int row_stride, int col0, int pos,
                                                         const u32x4 (&r)[4]) {
#pragma unroll
  for (int x = 0; x < 4; ++x)
    *reinterpret_cast<u32x4*>(tile + (col0 + x) * row_stride + pos) = u32x4{r[0][x], r[1][x], r[2][x], r[3][x]};
}

template <>
__device__ __forceinline__ void write_transposed4<__bf16>(__bf16* tile, int row_stride, int col0, int pos,
                                                          const u32x4 (&r)[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // element 2w sits in the low half of dword w, element 2w+1 in the high half
    const uint32_t lo0 = (r[0][w] & 0xffffu) | (r[1][w] << 16);
    const uint32_t hi0 = (r[2][w] & 0xffffu) | (r[3][w] << 16);
    const uint32_t lo1 = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
    const uint32_t hi1 = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
    *reinterpret_cast<u32x2*>(tile + (col0 + 2 * w) * row_stride + pos) = u32x2{lo0, hi0};
    *reinterpret_cast<u32x2*>(tile + (col0 + 2 * w + 1) * row_stride + pos) = u32x2{lo1, hi1};
  }
}

// fp16 moves the same 16-bit patterns as bf16.
template <>
__device__ __forceinline__ void write_transposed4<_Float16>(_Float16* tile, int row_stride, int col0, int pos,
                                                            const u32x4 (&r)[4]) {
  write_transposed4<__bf16>(reinterpret_cast<__bf16*>(tile), row_stride, col0, pos, r);
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Grouped-query attention: query head h of sequence b reads key/value head
// h / G (G = H / H_kv query heads per key/value head); the kernels pass that
// head with heads = H_kv to seq_rows below.
//
// Where the rows of one (sequence, head) live.  Fixed-length batches
// ([B, heads, N, d], cu == nullptr): head (b, h) starts at row
// (b*heads + h)*N and has N rows.  Packed ragged batches ([heads, T, d] with
// sequence offsets cu[0..B]): it starts at row h*T + cu[b] and has
// cu[b+1] - cu[b] rows.  Offsets are clamped to [0, T] and the length to
// Nmax, so inconsistent offsets give wrong rows but never an access outside
// the tensors.
// Non-causal tiles all cost the same, so a grid may visit a head's tiles
// together: workgroups are dealt to the 8 XCDs round-robin, and this order
// gives XCD x the tiles of heads x, x+8, ... one head after the other, so
// the K/V rows all of a head's query tiles read stay in that XCD's L2.
// (Causal grids keep the heaviest-first order instead.)
struct TileIdx {
  int tile, head;
};
__device__ __forceinline__ TileIdx xcd_head_major(int lin, int heads, int tiles) {
  if (heads % 8 != 0) return TileIdx{lin / heads, lin % heads};
  const int x = lin % 8, s = lin / 8;
  return TileIdx{s % tiles, (s / tiles) * 8 + x};
}

// Causal tiles cost different amounts, and a grid that runs the heaviest
// tiles of all heads first (heads fastest) leaves nothing long for the end.
// It also keeps tiles of every head live at once, heads / 8 of them on each
// XCD.  From 256 (sequence, head) pairs up (32 per XCD) their K/V rows no
// longer stay in the caches, and that order pays more in re-fetched rows
// than it saves in balance.  Measured, bf16 d = 128 causal: B16 H16 N4096
// forward 1.57 -> 1.23 ms and a packed batch of 16 sequences x 16 heads
// 0.64 -> 0.57 ms with the order below; with 64 heads it is 11-15 % slower,
// with 128 even, and at d = 64 with 256 heads even.  From that size up the
// grid visits a head's tiles together: the workgroups dealt to XCD x (every
// eighth one) take heads x, x + 8, ... one after the other, each head's
// tiles heaviest first.  What is counted is the distinct K/V working sets a
// grid streams: (sequence, key/value head) pairs for the forward and dQ
// grids, whose query heads share their group's K/V, and (piece, sequence,
// key/value head) triples for a dK/dV grid.
constexpr int kHeadGroupedHeads = 256;
struct CausalOrder {
  int rank, head;  // cost rank of the tile (0 = heaviest), (sequence, head)
};
__device__ __forceinline__ CausalOrder causal_order(int lin, int heads, int tiles, bool grouped) {
  if (grouped && heads % 8 == 0) {
    const int x = lin % 8, s = lin / 8;
    return CausalOrder{s % tiles, (s / tiles) * 8 + x};
  }
  return CausalOrder{lin / heads, lin % heads};
}

// Launch rank -> cost rank of a causal grid's tiles (cost rank 0 = the
// heaviest tile).  A grid spanning many rounds of resident workgroups runs
// heaviest first, so nothing long is left for the end.  A grid of at most two
// workgroups per CU is placed in one go, its first half one per CU and its
// second half beside it in the same CU order; there the second half is
// reversed ("snake"), so each CU holds one heavy and one light tile instead
// of two heavy ones or two light ones.
__device__ __forceinline__ int causal_rank(int p, int n, bool snake) {
  if (!snake) return p;
  const int half = (n + 1) / 2;
  return p < half ? p : n - 1 - (p - half);
}

struct SeqRows {
  long long row0;
  int n;
};
__device__ __forceinline__ SeqRows seq_rows(const int* cu, int Nmax, int T, int b, int h, int heads) {
  SeqRows r;
  if (cu == nullptr) {
    r.row0 = ((long long)b * heads + h) * Nmax;
    r.n = Nmax;
  } else {
    const int s = min(max(cu[b], 0), T);
    const int e = min(max(cu[b + 1], s), T);
    r.row0 = (long long)h * T + s;
    r.n = min(e - s, Nmax);
  }
  return r;
}


// The value held by lane l ^ 32 (the other half of the wave), through the
// gfx950 half-swap of two registers: a VALU operation, where a shuffle would
// make a round trip through the LDS unit.  The swap exchanges the upper half
// of its first operand with the lower half of its second, so with both set
// to v the lower lanes find the partner's value in the second result and the
// upper lanes in the first.
__device__ __forceinline__ float swap_halves(float v, int lane) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (lane & 32) ? r[0] : r[1]);
}

// Row stride (in 4-byte words) for an LDS tile that is only read through
// transpose reads.  The 32 lanes that the LDS serves together take a 64-byte
// column block (16 banks) from each of 4 consecutive rows, so the row starts
// stride*k mod 64 (k = 1..3) must keep those 16-bank windows apart.  Returns
// the smallest stride >= row_words that does.
constexpr int tr_stride_words(int row_words) {
  for (int s = row_words;; ++s) {
    bool ok = true;
    for (int k = 1; k < 4 && ok; ++k) {
      const int d = (s * k) % 64;
      if (d < 16 || d > 48) ok = false;
    }
    if (ok) return s;
  }
}

// Row stride (in 4-byte words) for an LDS tile whose rows hold `row_words`
// words and that is read both ways: 16 lanes reading 16 B from 16
// consecutive rows (row-contiguous MFMA operands) need (stride/4) odd, so the
// rows start on 16 distinct 4-bank groups of the 64 banks; 16 lanes of a
// transpose read touch 4 consecutive rows x 8 words, which need the four
// 8-bank windows stride*k mod 64 (k = 0..3) to be disjoint.  Returns the
// smallest stride >= row_words meeting both.
constexpr int lds_stride_words(int row_words) {
  for (int s = row_words;; ++s) {
    if (s % 4 != 0 || (s / 4) % 2 == 0) continue;
    bool ok = true;
    for (int a = 0; a < 4 && ok; ++a)
      for (int b = a + 1; b < 4 && ok; ++b) {
        const int d = ((s * b - s * a) % 64 + 64) % 64;
        if (d < 8 || d > 56) ok = false;
      }
    if (ok) return s;
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// A-operand fragment of chunk t for a product that contracts over the ROWS of
// a row-major LDS tile (the transposed operand V^T, Q^T, dO^T, K^T, ...).
// Lane (l32, h) supplies output row m = cb + l32 (a tile column) and the
// contraction slots of chunk t of the 32-row block starting at tile row rb,
// numbered exactly as pack_chunk numbers the accumulator rows it pairs with:
//   bf16: slots 0-3 = rows rb+16t+4h+0..3, slots 4-7 = rows rb+16t+8+4h+0..3;
//   fp32: slot e    = row  rb+8t+4h+e.
// bf16 uses the gfx950 LDS transpose read ds_read_b64_tr_b16: inside each
// 16-lane group, input lane j supplies the 8 bytes at row (j/4), columns
// 4*(j%4)..+3 of a 4x16 block and output lane i receives column i of all four
// rows.  Two such reads (rows +0..3 and +8..11) fill the 8 slots.  The bf16
// tile needs cb+32 readable columns per row (padding may supply them); the
// fp32 path reads column cb + (l32 & cmask) so narrow tiles stay in bounds.
template <typename T>
__device__ __forceinline__ u32x4 load_rowcontract(const T* tile, int stride, int rb, int t, int cb, int cmask,
                                                  int lane);

template <>
__device__ __forceinline__ u32x4 load_rowcontract<__bf16>(const __bf16* tile, int stride, int rb, int t, int cb,
                                                          int /*cmask*/, int lane) {
  const int h = lane >> 5, j = lane & 15;
  const int row = rb + 16 * t + 4 * h + (j >> 2);
  const int col = cb + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const __bf16* p = tile + row * stride + col;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * stride));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(u32x4, both);
}

template <>
__device__ __forceinline__ u32x4 load_rowcontract<_Float16>(const _Float16* tile, int stride, int rb, int t, int cb,
                                                            int cmask, int lane) {
  return load_rowcontract<__bf16>(reinterpret_cast<const __bf16*>(tile), stride, rb, t, cb, cmask, lane);
}

template <>
__device__ __forceinline__ u32x4 load_rowcontract<float>(const float* tile, int stride, int rb, int t, int cb,
                                                         int cmask, int lane) {
  const int h = lane >> 5, l32 = lane & 31;
  const float* p = tile + (rb + 8 * t + 4 * h) * stride + cb + (l32 & cmask);
  return as_u32x4(f32x4{p[0], p[stride], p[2 * stride], p[3 * stride]});
}

__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace fa2
