// fa2_fwd.hip -- FlashAttention-2 forward pass for gfx950.
//
// The article "Revolutionizing Web-Based AI: How a Plain JavaScript Prototype
// Paved the Way for High-Performance WebGPU Flash Attention 2" (section
// "Translating to WGSL and Optimizing Passes") gives the shape of the pass:
// one workgroup per (batch, head, query tile), keys and values visited in
// blocks, the online-softmax state kept in registers, no N x N matrix in
// global memory.  Section "Memory Bandwidth Optimization" adds that the
// softmax reduction is built up block by block.  What follows is that pass
// laid out for CDNA4.
//
// Two kernels follow: fwd_kernel for every type and head size, and
// fwd_pp_kernel, a leaner schedule of the same pass for the 16-bit types
// (bf16, fp16) at d = 128.  Both serve fixed-length batches ([B, H, N, d]),
// packed ragged batches ([H, T, d] with sequence offsets) and grouped-query
// heads; fwd_kernel also serves decoding for the types and head sizes the
// split-cache decode kernel does not cover (a key length of its own, the
// queries being the last positions).
//
// Workgroup: 4 waves x 32 query rows = a 128-row query tile.  Each wave
// computes the TRANSPOSED score block S^T = K Q^T (keys x queries) on MFMA,
// so every lane owns one query column: its running max m and sum l are
// plain per-lane registers, the row reduction is a loop over the lane's own
// accumulators plus one half-swap with lane l^32, and the exponentiated block
// is already laid out as the B operand of O^T += V^T P^T.  K and V tiles are
// staged row-major in LDS (global loads of tile j+1 are issued before tile j
// is computed and land in the other buffer; one barrier per tile).  The V^T
// operand is read with the gfx950 LDS transpose read, so nothing is ever
// written transposed.
//
// Causal: query tiles are launched heaviest first, key tiles past the
// diagonal are never visited, 32-key blocks fully above a wave's rows are
// skipped, and the mask is only evaluated on blocks that straddle the
// diagonal or the ragged end of the sequence.
//
// Numerics: logits are accumulated in fp32 and scaled after the product
// (an input is never pre-scaled); the softmax runs in base 2 with
// scale*log2(e) folded into one FMA.  The running max only moves when the
// block max exceeds it by more than kSlack (base-2 units), so the O rescale
// is skipped in most tiles; weights are then at most 2^kSlack, harmless in
// fp32 and the 16-bit types.  At the end O = acc / l and
// LSE = (m + log2 l) * ln 2.
#include "fa2_common.hpp"
#include "fa2_launch.hpp"
#include "fa2_swz.hpp"

namespace fa2 {

template <typename T, int D>
struct FwdTile {
  static constexpr int NW = 4;
  static constexpr int BR = 32 * NW;                   // query rows per workgroup
  static constexpr int BC = sizeof(T) == 2 ? 64 : 32;  // keys per LDS tile
  static constexpr int CH = Elt<T>::CH;
  static constexpr int KS = D + CH;  // K row stride: 16-byte pad, conflict-free row reads
  // V row stride: V is only read through transpose reads (bf16), which need
  // 4 consecutive rows on disjoint 16-bank windows (and at least 32 columns
  // per row, which is what a read spans); fp32 reads 4 rows per lane.
  static constexpr int VS = sizeof(T) == 2 ? 2 * tr_stride_words((D >= 32 ? D : 32) / 2) : D + 4;
  static constexpr int NB = D >= 32 ? D / 32 : 1;  // 32-row output blocks over d
  static constexpr int CMASK = (D >= 32 ? 32 : D) - 1;
  static constexpr int DCH = D / (2 * CH);  // chunks of a contraction over d
  static constexpr int NJB = BC / 32;       // 32-key blocks per tile
  static constexpr int CPB = 16 / CH;       // chunks per 32-key block
  static constexpr int ROW_CH = D / CH;     // 16-byte chunks per row
  static constexpr int CHUNKS = BC * ROW_CH;
  static constexpr int PER_T = (CHUNKS + 255) / 256;
};

// SPLIT = 1: four waves, each with its own 32 query rows, walk the key
// tiles together.  SPLIT = 2 (fp32 grids too small to fill the device): the
// 4 waves form 2 query groups of 32 rows, and the 2 waves of a group take
// alternate key tiles (each step brings in one tile per wave), so the
// longest walk is halved; at the end each pair merges its (max, sum, O) in
// LDS with the same rescaling as the online softmax.  SPLIT = 4 (the same
// grids at d <= 32): one query group of 32 rows whose 4 waves take every
// fourth key tile, with one LDS buffer (the next step's tiles wait in
// registers until every wave is done with the current ones), so four
// workgroups fit on a CU; the four walks merge in LDS in wave order.
template <typename T, int D, bool CAUSAL, int SPLIT>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                     const T* __restrict__ V, T* __restrict__ O,
                                                     float* __restrict__ LSE, int Nmax, int BH, int num_qt,
                                                     float sl2, int H, int G, const int* __restrict__ cu,
                                                     int Ttot, int Nk, int snake) {
  using C = FwdTile<T, D>;
  constexpr int CH = C::CH, BC = C::BC, KS = C::KS, VS = C::VS;
  constexpr int BR = 32 * C::NW / SPLIT;  // query rows per workgroup
  constexpr int NBUF = SPLIT == 4 ? 1 : 2;  // LDS buffers of tiles
  constexpr int CHUNKS = SPLIT * C::CHUNKS;
  constexpr int PER_T = (CHUNKS + 255) / 256;
  __shared__ __attribute__((aligned(16))) T Ks[NBUF][SPLIT * BC * KS];
  __shared__ __attribute__((aligned(16))) T Vs[NBUF][SPLIT * BC * VS];
  // Merge area of the four-walk split (three walks' max, sums and
  // accumulators): the K tiles when they are large enough, else its own.
  constexpr int XSLOT = C::NB * 16 * 64 + 2 * 64;
  constexpr int XM = (SPLIT == 4 && 3 * XSLOT * sizeof(float) > sizeof(T) * NBUF * SPLIT * BC * KS) ? 3 * XSLOT : 1;
  __shared__ __attribute__((aligned(16))) float Xm[XM];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int qg = w / SPLIT;  // query group of this wave
  const int kp = w % SPLIT;  // which of each step's SPLIT key tiles it takes
  const int lin = blockIdx.x;
  const int qt = CAUSAL ? (num_qt - 1 - causal_rank(lin / BH, num_qt, snake != 0)) : (lin / BH);
  const int bh = lin % BH;
  const SeqRows sq = seq_rows(cu, Nmax, Ttot, bh / H, bh % H, H);
  const int N = sq.n;  // this sequence's length (query rows)
  // Keys: the same rows, or (decoding, Nk > 0) a cache of Nk rows per
  // key/value head whose last N positions are the queries, so with the
  // causal mask query i keeps keys j <= i + coff.
  const int Nkv = Nk > 0 ? Nk : N;
  const int coff = Nkv - N;
  const long long kv_row0 = Nk > 0 ? ((long long)(bh / H) * (H / G) + (bh % H) / G) * Nk
                                   : seq_rows(cu, Nmax, Ttot, bh / H, (bh % H) / G, H / G).row0;
  const size_t base = (size_t)sq.row0 * D;
  const size_t kv_base = (size_t)kv_row0 * D;
  const T* Qh = Q + base;
  const T* Kh = K + kv_base;
  const T* Vh = V + kv_base;
  const int q0 = qt * BR;
  if (q0 >= N) return;          // a tile past a shorter packed sequence
  const int qw = q0 + 32 * qg;  // first query row of this wave
  const int qi = qw + l32;      // query row (column of S^T) owned by this lane

  // Q^T as the B operand of S^T = K Q^T: lane holds its query row, chunked
  // over d.  Rows past N load row N-1 (finite) and are never stored.
  u32x4 qf[C::DCH];
  {
    const T* qrow = Qh + (size_t)min(qi, N - 1) * D + h * CH;
#pragma unroll
    for (int c = 0; c < C::DCH; ++c) qf[c] = load16(qrow + c * 2 * CH);
  }
  negate_fragments_if<T>(qf, C::DCH, sl2);

  const int kv_end = CAUSAL ? min(Nkv, q0 + BR + coff) : Nkv;
  const int n_kt = (kv_end + BC - 1) / BC;
  const int n_st = (n_kt + SPLIT - 1) / SPLIT;  // steps of SPLIT tiles

  // Step loads: tiles SPLIT*st .. SPLIT*st + SPLIT - 1, rows past Nkv (and
  // tiles past the last) load row Nkv-1; those keys are masked to -inf or
  // never visited, so their (finite) values never reach the output.
  u32x4 kr[PER_T], vr[PER_T];
  auto load_step = [&](int st) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int c = tid + 256 * u;
      if (c < CHUNKS) {
        const int j = c / C::CHUNKS, cc = c % C::CHUNKS;
        const size_t off = (size_t)min((SPLIT * st + j) * BC + cc / C::ROW_CH, Nkv - 1) * D + (cc % C::ROW_CH) * CH;
        kr[u] = load16(Kh + off);
        vr[u] = load16(Vh + off);
      }
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int c = tid + 256 * u;
      if (c < CHUNKS) {
        const int j = c / C::CHUNKS, cc = c % C::CHUNKS;
        const int row = cc / C::ROW_CH, col = (cc % C::ROW_CH) * CH;
        store16(&Ks[buf][(j * BC + row) * KS + col], kr[u]);
        store16(&Vs[buf][(j * BC + row) * VS + col], vr[u]);
      }
    }
  };

  f32x16 o[C::NB];
#pragma unroll
  for (int b = 0; b < C::NB; ++b) o[b] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled logits, base-2 units
  float l_run = 0.f;        // this lane half's share of the running sum

  load_step(0);
  store_step(0);
  __syncthreads();

  // One key tile of this wave.  Each 32-key block runs its own
  // online-softmax update, so a block's exponentials depend only on its own
  // scores and the next block's score MFMAs can run under them.
  auto tile = [&](int kt, const T* ks, const T* vs, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const int kb0 = kt * BC;
    // 32-key blocks of this tile that hold a key this wave may see.
    const int last_key = CAUSAL ? min(qw + 31 + coff, Nkv - 1) : Nkv - 1;
    const int nlive = MASKED ? (last_key < kb0 ? 0 : min(C::NJB, (last_key - kb0) / 32 + 1)) : C::NJB;

    f32x16 s[C::NJB];
#pragma unroll
    for (int jb = 0; jb < C::NJB; ++jb) {
      if (jb < nlive) {
        s[jb] = f32x16{};
        const T* krow = ks + (32 * jb + l32) * KS + h * CH;
#pragma unroll
        for (int c = 0; c < C::DCH; ++c) mfma_chunk<T>(s[jb], load16(krow + c * 2 * CH), qf[c]);
      }
    }
#pragma unroll
    for (int jb = 0; jb < C::NJB; ++jb) {
      if (jb < nlive) {
        const int kb = kb0 + 32 * jb;
        if (MASKED) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = kb + acc_row(r, h);
            s[jb][r] = ((CAUSAL & (j > qi + coff)) | (j >= Nkv)) ? -INFINITY : s[jb][r];  // a select
          }
        }
        float mx = s[jb][0];
#pragma unroll
        for (int r = 1; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[jb][r], s[jb][r + 1 < 16 ? r + 1 : r]));
        mx = fmaxf(mx, swap_halves(mx, lane));
        const float m_cand = mx * sl2;
        const bool grow = m_cand > m_run + kSlack;
        if (__any(grow)) {
          const float m_new = grow ? m_cand : m_run;
          // 0 on a lane's first visible keys; exactly 1 where the max stays.
          const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int b = 0; b < C::NB; ++b) o[b] *= alpha;
        }
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
        // The row sum is taken over the fp32 weights (summing the rounded
        // bf16 weights instead costs LSE accuracy: ~1e-4 relative).
        float l_blk = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[jb][r] = __builtin_amdgcn_exp2f(fmaf(s[jb][r], sl2, neg_m));
          l_blk += s[jb][r];
        }
        l_run += l_blk;
#pragma unroll
        for (int t = 0; t < C::CPB; ++t) {
          const u32x4 pb = pack_chunk<T>(s[jb], t);
#pragma unroll
          for (int b = 0; b < C::NB; ++b)
            mfma_chunk<T>(o[b], load_rowcontract<T>(vs, VS, 32 * jb, t, 32 * b, C::CMASK, lane), pb);
        }
      }
    }
  };
  // Key tiles wholly below every row of this query tile and wholly before Nkv
  // need no mask; the diagonal and ragged tiles come last.
  const int kt_full = min(n_kt, CAUSAL ? min(q0 + coff, Nkv) / BC : Nkv / BC);
  if constexpr (SPLIT == 1) {
    auto step = [&](int kt, auto masked) {
      const bool more = kt + 1 < n_kt;
      if (more) load_step(kt + 1);
      tile(kt, Ks[kt & 1], Vs[kt & 1], masked);
      if (more) store_step((kt + 1) & 1);
      __syncthreads();
    };
    int kt = 0;
    for (; kt < kt_full; ++kt) step(kt, BoolC<false>{});
    for (; kt < n_kt; ++kt) step(kt, BoolC<true>{});
  } else {
    for (int st = 0; st < n_st; ++st) {
      const bool more = st + 1 < n_st;
      if (more) load_step(st + 1);
      const int kt = SPLIT * st + kp;  // this wave's tile (uniform per wave)
      const T* ks = &Ks[(st & 1) % NBUF][kp * BC * KS];
      const T* vs = &Vs[(st & 1) % NBUF][kp * BC * VS];
      if (kt < kt_full)
        tile(kt, ks, vs, BoolC<false>{});
      else if (kt < n_kt)
        tile(kt, ks, vs, BoolC<true>{});
      if constexpr (NBUF == 1) {
        __syncthreads();  // every wave is done with the one buffer
        if (more) store_step(0);
      } else {
        if (more) store_step((st + 1) & 1);
      }
      __syncthreads();
    }
  }

  if constexpr (SPLIT == 4) {
    // Merge the four walks: waves 1..3 leave their max, sums and accumulators
    // in LDS (the last step ended with a barrier), wave 0 (which walked key
    // 0, so its max is finite) combines them in wave order.
    constexpr int SLOT = XSLOT;  // floats per walk
    float* xo = XM > 1 ? Xm : reinterpret_cast<float*>(&Ks[0][0]);
    if (kp > 0) {
      float* my = xo + (kp - 1) * SLOT;
#pragma unroll
      for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) my[(16 * b + r) * 64 + lane] = o[b][r];
      my[C::NB * 16 * 64 + lane] = m_run;
      my[C::NB * 16 * 64 + 64 + lane] = l_run;
    }
    __syncthreads();
    if (kp > 0) return;
    float mp[3], lp[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      mp[i] = xo[i * SLOT + C::NB * 16 * 64 + lane];
      lp[i] = xo[i * SLOT + C::NB * 16 * 64 + 64 + lane];
    }
    const float m = fmaxf(fmaxf(m_run, mp[0]), fmaxf(mp[1], mp[2]));
    const float a0 = __builtin_amdgcn_exp2f(m_run - m);
    float ap[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) ap[i] = mp[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mp[i] - m);
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = o[b][r] * a0;
#pragma unroll
        for (int i = 0; i < 3; ++i) x += xo[i * SLOT + (16 * b + r) * 64 + lane] * ap[i];
        o[b][r] = x;
      }
    float l = l_run * a0;
#pragma unroll
    for (int i = 0; i < 3; ++i) l += lp[i] * ap[i];
    l_run = l;
    m_run = m;
  }
  if constexpr (SPLIT == 2) {
    // Merge the two walks of each query group: the odd wave leaves its max,
    // sums and accumulators in LDS (the tiles are no longer read: the last
    // step ended with a barrier), the even one combines them.  The even wave
    // walked key 0, so its max is finite.
    constexpr int SLOT = C::NB * 16 * 64 + 2 * 64;  // floats per query group
    static_assert(2 * SLOT * sizeof(float) <= sizeof(Ks), "merge area");
    float* xo = reinterpret_cast<float*>(&Ks[0][0]) + qg * SLOT;
    if (kp == 1) {
#pragma unroll
      for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(16 * b + r) * 64 + lane] = o[b][r];
      xo[C::NB * 16 * 64 + lane] = m_run;
      xo[C::NB * 16 * 64 + 64 + lane] = l_run;
    }
    __syncthreads();
    if (kp == 1) return;
    const float m1 = xo[C::NB * 16 * 64 + lane];
    const float l1 = xo[C::NB * 16 * 64 + 64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[b][r] = o[b][r] * a0 + xo[(16 * b + r) * 64 + lane] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_run = m;
  }

  const float l_tot = l_run + swap_halves(l_run, lane);
  if (qi < N) {
    const float inv = 1.0f / l_tot;
    T* Oi = O + base + (size_t)qi * D;
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * b + 8 * g + 4 * h;
        if (d0 < D)
          store4<T>(Oi + d0, o[b][4 * g] * inv, o[b][4 * g + 1] * inv, o[b][4 * g + 2] * inv,
                    o[b][4 * g + 3] * inv);
      }
    }
    if (h == 0) LSE[sq.row0 + qi] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// Forward for the 16-bit types at d = 128 and d = 64.  Same pass as
// fwd_kernel, organised around 32-key blocks that reach LDS through direct
// loads into a ring of 4 block slots (K and V, unpadded swizzled rows:
// 256-byte rows swizzled by swz, 128-byte rows by swz64), issued 3 blocks
// ahead, one barrier per block.  Within a wave the score products of block b+1 are
// issued before the softmax of block b, so the matrix cores have work while
// the exponentials of block b run; then P V of block b follows.
//
// On gfx950 a wave64 fp32 FMA occupies its SIMD for 4 clocks, an exp for 8
// and a 32x32x16 MFMA for 32, and vector work only partly hides under the
// products of the same or a neighbouring wave.  So the per-block vector
// instruction count is what bounds this kernel next to the products, and it
// is kept near the softmax's own work: lane offsets for every LDS fragment
// and direct load are computed once, block slots are compile-time (the
// block loop is unrolled over the ring), the row offset of a load goes in
// the uniform buffer offset, and the rare running-max rescale is a real
// branch.
namespace fpp {
constexpr int BR = 128;        // query rows per workgroup (4 waves x 32)
constexpr int KB = 32;         // keys per block
// Workgroups per CU: at d = 64 three fit (168 registers, 3 x 32 KB of LDS).
constexpr int occupancy(int D) { return D == 64 ? 3 : 2; }
}  // namespace fpp

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, fpp::occupancy(D)) void fwd_pp_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                        const T* __restrict__ V, T* __restrict__ O,
                                                        float* __restrict__ LSE, int Nmax, int BH, int num_qt,
                                                        float sl2, int H, int G, const int* __restrict__ cu,
                                                        int Ttot) {
  using namespace tiles;
  static_assert(D == 128 || D == 64, "fwd_pp_kernel: d = 128 or 64");
  constexpr int KB = fpp::KB, BLK_E = KB * D;
  constexpr int CH = 8, DCH = D / 16, NB = D / 32;
  constexpr int ROWB = 2 * D;           // bytes per LDS row
  constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  constexpr int RPL = 1024 / ROWB;      // rows per 1-KB wave load
  constexpr int LPT = KB / RPL;         // loads per tensor per block
  constexpr int LPW = 2 * LPT / 4;      // loads per wave per block
  constexpr int R = 4, PF = R - 1;  // ring slots, blocks loaded ahead
  __shared__ __attribute__((aligned(16))) T Ks[R][BLK_E];
  __shared__ __attribute__((aligned(16))) T Vs[R][BLK_E];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int lin = blockIdx.x;
  // Causal: heaviest query tiles first (causal_order); otherwise a head's
  // tiles together on one XCD.
  TileIdx ti;
  if (CAUSAL) {
    const CausalOrder co = causal_order(lin, BH, num_qt, BH / G >= kHeadGroupedHeads);
    ti = TileIdx{num_qt - 1 - co.rank, co.head};
  } else {
    ti = xcd_head_major(lin, BH, num_qt);
  }
  const int qt = ti.tile;
  const int bh = ti.head;
  const SeqRows sq = seq_rows(cu, Nmax, Ttot, bh / H, bh % H, H);
  const int N = sq.n;  // this sequence's length
  const size_t base = (size_t)sq.row0 * D;
  const T* Qh = Q + base;
  const int q0 = qt * fpp::BR;
  if (q0 >= N) return;  // a tile past a shorter packed sequence
  const int qw = q0 + 32 * w;  // first query row of this wave
  const int qi = qw + l32;     // query row (column of S^T) owned by this lane
  // Waves 0-1 load K rows, waves 2-3 V rows: load u of wave w is number
  // q = LPW w + u, rows RPL (q % LPT) .. + RPL - 1 of the block.
  const long long kv_row0 = seq_rows(cu, Nmax, Ttot, bh / H, (bh % H) / G, H / G).row0;
  const u32x4 rsrc = make_rsrc((w < 2 ? K : V) + (size_t)kv_row0 * D, (unsigned)N * D * 2);
  T* const dst0 = w < 2 ? &Ks[0][0] : &Vs[0][0];

  const int kv_end = CAUSAL ? min(N, q0 + fpp::BR) : N;
  const int nb = (kv_end + KB - 1) / KB;

  // Per-lane constants: direct-load offsets within a block, and the LDS
  // fragment offsets (K row fragments by chunk, V transpose fragments by
  // column block and half); block slots and the t half are immediates.
  auto swz_row = [](int r) { return D == 128 ? swz(r) : swz64(r); };
  int voff[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int r = RPL * ((LPW * w + u) % LPT) + lane / CPR;
    voff[u] = r * ROWB + (((lane % CPR) ^ swz_row(r)) << 4);
  }
  const SwzOffsets so = D == 128 ? swz_offsets(lane) : swz_offsets64(lane);
  int kofs[DCH], vofs0[NB], vofs1[NB];
#pragma unroll
  for (int c = 0; c < DCH; ++c) kofs[c] = so.rofs ^ (c << 5);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    vofs0[b] = so.tofs0 + ((b ^ so.kk) << 6);
    vofs1[b] = so.tofs1 + ((b ^ so.kk) << 6);
  }

  // Block kb into slot (its rows past N read row N-1; they are masked).
  auto issue = [&](int kb, int slot) {
    const int row0 = kb * KB;
    T* dst = dst0 + slot * BLK_E;
    if (row0 + KB <= N) {
#pragma unroll
      for (int u = 0; u < LPW; ++u) bload16(rsrc, voff[u], row0 * ROWB, dst + ((LPW * w + u) % LPT) * 512);
    } else {
#pragma unroll
      for (int u = 0; u < LPW; ++u) {
        const int r = RPL * ((LPW * w + u) % LPT) + lane / CPR;
        bload16(rsrc, min(row0 + r, N - 1) * ROWB + (voff[u] & (ROWB - 1)), 0,
                dst + ((LPW * w + u) % LPT) * 512);
      }
    }
  };

  u32x4 qf[DCH];
  {
    const T* qrow = Qh + (size_t)min(qi, N - 1) * D + h * CH;
#pragma unroll
    for (int c = 0; c < DCH; ++c) qf[c] = load16(qrow + c * 2 * CH);
  }
  negate_fragments_if<T>(qf, DCH, sl2);
#pragma unroll
  for (int b = 0; b < PF; ++b)
    if (b < nb) issue(b, b);
  wait_vmem();
  __syncthreads();

  // S^T = K Q^T for the block in slot (keys x this wave's 32 queries).
  auto scores = [&](int slot) {
    f32x16 s = f32x16{};
    const char* kb_ = reinterpret_cast<const char*>(Ks[slot]);
#pragma unroll
    for (int c = 0; c < DCH; ++c) mfma_chunk<T>(s, lds16(kb_, kofs[c]), qf[c]);
    return s;
  };

  f32x16 o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled logits, base-2 units
  float l_run = 0.f;        // this lane half's share of the running sum

  // Block kb (slot SLOT): scores of block kb+1 into s_nx, softmax and P V
  // of block kb from s.
  auto block = [&](auto slotc, int kb, auto masked, f32x16& s, f32x16& s_nx) {
    constexpr int SLOT = decltype(slotc)::value;
    constexpr bool MASKED = decltype(masked)::value;
    const bool ahead = kb + PF < nb;
    if (ahead) issue(kb + PF, (SLOT + PF) % R);
    const int k0 = kb * KB;
    if (MASKED) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = k0 + acc_row(r, h);
        s[r] = ((CAUSAL & (j > qi)) | (j >= N)) ? -INFINITY : s[r];
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[r], s[r + 1 < 16 ? r + 1 : r]));
    mx = fmaxf(mx, swap_halves(mx, lane));
    const float m_cand = mx * sl2;
    const bool grow = m_cand > m_run + kSlack;
    if (__builtin_expect(__any(grow), 0)) {
      // Rare (the max moves by more than kSlack): kept as a real branch; the
      // empty asm stops the compiler from turning it into 64 unconditional
      // multiplies by a selected 1.
      asm volatile("");
      const float m_new = grow ? m_cand : m_run;
      const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b] *= alpha;
    }
    // Scores of the next block (the slot past the last block holds stale
    // data; that result is never used).
    s_nx = scores((SLOT + 1) % R);
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    float l_blk = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, neg_m));
      l_blk += s[r];
    }
    l_run += l_blk;
    const char* vb_ = reinterpret_cast<const char*>(Vs[SLOT]);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pb = pack_chunk<T>(s, t);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        mfma_chunk<T>(o[b], tr_frag(vb_, vofs0[b] + t * 16 * ROWB, vofs1[b] + t * 16 * ROWB), pb);
    }
    // Blocks kb+1 .. kb+PF-1 must be in LDS for the next block; the LPW
    // loads of block kb+PF issued above may stay in flight.
    if (ahead)
      wait_vmem_n<LPW>();
    else
      wait_vmem();
    __syncthreads();
  };
  // Blocks wholly below every row of this query tile and before N need no
  // mask; the diagonal and ragged blocks come last.
  const int nb_full = min(nb, CAUSAL ? min(q0, N) / KB : N / KB);
  f32x16 s0 = scores(0), s1;
  int kb = 0;
  for (; kb + 4 <= nb_full; kb += 4) {
    block(IntC<0>{}, kb, BoolC<false>{}, s0, s1);
    block(IntC<1>{}, kb + 1, BoolC<false>{}, s1, s0);
    block(IntC<2>{}, kb + 2, BoolC<false>{}, s0, s1);
    block(IntC<3>{}, kb + 3, BoolC<false>{}, s1, s0);
  }
  // The rest (at most 3 full blocks, then the masked ones), slot by slot.
  for (; kb < nb; ++kb) {
    switch (kb & 3) {
      case 0: block(IntC<0>{}, kb, BoolC<true>{}, s0, s1); break;
      case 1: block(IntC<1>{}, kb, BoolC<true>{}, s0, s1); break;
      case 2: block(IntC<2>{}, kb, BoolC<true>{}, s0, s1); break;
      default: block(IntC<3>{}, kb, BoolC<true>{}, s0, s1); break;
    }
    s0 = s1;
  }

  const float l_tot = l_run + swap_halves(l_run, lane);
  if (qi < N) {
    const float inv = 1.0f / l_tot;
    T* Oi = O + base + (size_t)qi * D;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * b + 8 * g + 4 * h;
        store4<T>(Oi + d0, o[b][4 * g] * inv, o[b][4 * g + 1] * inv, o[b][4 * g + 2] * inv,
                  o[b][4 * g + 3] * inv);
      }
    }
    if (h == 0) LSE[sq.row0 + qi] = (m_run + log2f(l_tot)) * kLn2;
  }
}


// Grids of at most this many workgroups (two per CU) are placed in one go:
// they take the snake order of causal_rank, and fp32 ones below it split
// their walks.
constexpr long long kFwdSplitGrid = 512;

template <typename T, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  if constexpr (sizeof(T) == 2 && (D == 128 || D == 64)) {
    // (Decoding through this launcher, Nk > 0, takes the generic kernel.)
    if (a.Nk == 0 && !force_generic_kernels()) {
      const int BH = a.B * a.H;
      const int num_qt = (a.N + fpp::BR - 1) / fpp::BR;
      const long long blocks = (long long)num_qt * BH;
      if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL((fwd_pp_kernel<T, D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                         static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                         static_cast<T*>(a.o), a.lse, a.N, BH, num_qt, a.scale * kLog2e, a.H, a.H / a.Hkv, a.cu,
                         a.T);
      return hipGetLastError();
    }
  }
  using C = FwdTile<T, D>;
  const int BH = a.B * a.H;
  const float sl2 = a.scale * kLog2e;
  const long long blocks4 = (long long)((a.N + C::BR - 1) / C::BR) * BH;
  if constexpr (sizeof(T) == 4 && D <= 64) {
    // fp32 grids of fewer than two 128-row tiles per CU: split each walk
    // over two waves (half-size query tiles, so twice the workgroups), or at
    // d <= 32, where four one-buffer workgroups fit on a CU, over four
    // (quarter-size query tiles).
    if (a.Nk == 0 && blocks4 < kFwdSplitGrid) {
      constexpr int SP = D <= 32 ? 4 : 2;
      const int num_qt = (a.N + C::BR / SP - 1) / (C::BR / SP);
      const long long blocks = (long long)num_qt * BH;
      hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, SP>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                         static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                         static_cast<T*>(a.o), a.lse, a.N, BH, num_qt, sl2, a.H, a.H / a.Hkv, a.cu, a.T, a.Nk,
                         (int)(blocks <= kFwdSplitGrid));
      return hipGetLastError();
    }
  }
  const int num_qt = (a.N + C::BR - 1) / C::BR;
  const long long blocks = blocks4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, 1>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                     static_cast<T*>(a.o), a.lse, a.N, BH, num_qt, sl2, a.H, a.H / a.Hkv, a.cu, a.T, a.Nk,
                     (int)(blocks <= kFwdSplitGrid));
  return hipGetLastError();
}

template <typename T, bool CAUSAL>
static hipError_t launch_fwd_d(const FwdArgs& a) {
  switch (a.d) {
    case 16: return launch_fwd_t<T, 16, CAUSAL>(a);
    case 32: return launch_fwd_t<T, 32, CAUSAL>(a);
    case 64: return launch_fwd_t<T, 64, CAUSAL>(a);
    case 128: return launch_fwd_t<T, 128, CAUSAL>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_forward(const FwdArgs& a) {
  if (a.dtype == kBF16)
    return a.causal ? launch_fwd_d<__bf16, true>(a) : launch_fwd_d<__bf16, false>(a);
  if (a.dtype == kF16)
    return a.causal ? launch_fwd_d<_Float16, true>(a) : launch_fwd_d<_Float16, false>(a);
  return a.causal ? launch_fwd_d<float, true>(a) : launch_fwd_d<float, false>(a);
}

}  // namespace fa2
