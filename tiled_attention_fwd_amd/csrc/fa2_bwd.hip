// fa2_bwd.hip -- FlashAttention-2 backward pass for gfx950.
//
// The article "Revolutionizing Web-Based AI: How a Plain JavaScript Prototype
// Paved the Way for High-Performance WebGPU Flash Attention 2" (section
// "Translating to WGSL and Optimizing Passes", backward-pass bullet) states
// the one rule that shapes this pass: the attention weights are not read
// back from a cached matrix but rebuilt from Q, K and the log-sum-exp saved
// by the forward pass.  Its section "Numerical Stability and Loss Drift"
// names atomic reductions as an accepted source of rounding differences.
// The gradient formulas are those of softmax attention:
//   P = exp(scale*QK^T - LSE),  dV = P^T dO,  dP = dO V^T,
//   dS = P o (dP - D) with D_i = sum_j P_ij dP_ij = rowsum(dO o O),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Kernels, in stream order:
//   bwd_dq_kernel    stage 1: one workgroup per (batch, head, 128-query
//                    tile), shaped like the forward pass: S^T = K Q^T and
//                    dP^T = V dO^T on MFMA, so each lane owns one query and
//                    its LSE and D are scalars, then dQ^T += K^T dS^T.  It
//                    first computes D = rowsum(dO o O) (it holds the lane's
//                    dO row already and loads its O row; a row whose keys
//                    all lie in its first 32-key block takes sum_j P_ij dP_ij
//                    from that block instead) and LSE * log2(e) for its rows
//                    and writes both to the workspace for the dK/dV kernel.
//                    For the 16-bit types at d = 128 and 64, bwd_dq_pp_kernel
//                    runs the same pass over a ring of direct-loaded 32-key
//                    blocks, like fwd_pp_kernel.  Small fp32 grids pair the
//                    walks: 64-row workgroups whose two waves per row group
//                    take alternate key tiles and add their dQ in LDS.
//   bwd_dkdv_kernel  stage 2: one workgroup per (batch, head, 128-key tile);
//                    each of its 4 waves owns 32 keys and keeps K, V (as MFMA
//                    B operands) and its dK^T, dV^T accumulators in registers
//                    while it walks the query tiles: S = Q K^T and
//                    dP = dO V^T on MFMA, P and dS in fp32, then
//                    dV^T += dO^T P and dK^T += Q^T dS on MFMA, with P and dS
//                    fed straight from the accumulator layout and Q^T, dO^T
//                    read from the row-major LDS tiles by transpose reads.
//                    For bf16 and fp16 at d = 128, bwd_dkdv_d128_kernel
//                    runs the same pass with direct-to-LDS loads into
//                    swizzled tiles and two independent workgroups per CU;
//                    bwd_dkdv_d64_kernel does the same at d = 64.
//                    With grouped-query heads a workgroup walks every query
//                    head of its key/value head's group (or a 1/S share of
//                    them; in fp32, a 1/S share of the query tiles), and
//                    bwd_dkdv_reduce_kernel sums the S fp32 partials in a
//                    fixed order.  Small fp32 grids first pair the walks:
//                    64-key workgroups whose two waves per key group take
//                    alternate query steps and add dK, dV in LDS.
//   There is no third stage: dQ comes with stage 1.
// Every kernel takes its (sequence, head) rows from seq_rows, so fixed-length
// and packed ragged batches share them.
// The two halves recompute S and dP instead of exchanging dS, so dQ needs no
// atomics or fp32 accumulator and the result is deterministic.
// Causal: tiles start and stop at the diagonal, blocks entirely above it
// are skipped, and only blocks that straddle it (or the ragged end of the
// sequence) evaluate the mask.
#include "fa2_common.hpp"
#include "fa2_launch.hpp"
#include "fa2_swz.hpp"

namespace fa2 {

template <typename T>
__device__ __forceinline__ float dot_chunk(u32x4 a, u32x4 b);

template <>
__device__ __forceinline__ float dot_chunk<float>(u32x4 a, u32x4 b) {
  const f32x4 af = as_f32x4(a), bf = as_f32x4(b);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s = fmaf(af[e], bf[e], s);
  return s;
}

template <>
__device__ __forceinline__ float dot_chunk<__bf16>(u32x4 a, u32x4 b) {
  // bf16 -> fp32 is exact: the bf16 bits become the high half of the float.
  const f32x4 a_lo = as_f32x4(a << 16), a_hi = as_f32x4(a & 0xffff0000u);
  const f32x4 b_lo = as_f32x4(b << 16), b_hi = as_f32x4(b & 0xffff0000u);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s = fmaf(a_lo[e], b_lo[e], s);
    s = fmaf(a_hi[e], b_hi[e], s);
  }
  return s;
}

template <>
__device__ __forceinline__ float dot_chunk<_Float16>(u32x4 a, u32x4 b) {
  // v_dot2_f32_f16: fp16 products are exact in fp32.
  const f16x8 ah = __builtin_bit_cast(f16x8, a), bh = __builtin_bit_cast(f16x8, b);
  float s = 0.f;
  s = __builtin_amdgcn_fdot2(__builtin_shufflevector(ah, ah, 0, 1), __builtin_shufflevector(bh, bh, 0, 1), s, false);
  s = __builtin_amdgcn_fdot2(__builtin_shufflevector(ah, ah, 2, 3), __builtin_shufflevector(bh, bh, 2, 3), s, false);
  s = __builtin_amdgcn_fdot2(__builtin_shufflevector(ah, ah, 4, 5), __builtin_shufflevector(bh, bh, 4, 5), s, false);
  s = __builtin_amdgcn_fdot2(__builtin_shufflevector(ah, ah, 6, 7), __builtin_shufflevector(bh, bh, 6, 7), s, false);
  return s;
}

// D_i = sum_k dO_ik O_ik for the row a lane pair owns in the dQ kernels.
// Lane half h holds 16-byte chunks 2c + h (c < DCH) of the row; pc[c] is the
// dot product of chunk 2c + h.  The chunks are added pairwise at distances
// DCH/2, DCH/4, .., 1 within the lane, then the two halves' sums with one
// exchange: a fixed tree, the same for every kernel and launch.
template <int DCH>
__device__ __forceinline__ float row_dot(float (&pc)[DCH], int lane) {
#pragma unroll
  for (int o = DCH / 2; o >= 1; o /= 2)
#pragma unroll
    for (int c = 0; c < o; ++c) pc[c] = pc[c] + pc[c + o];
  return pc[0] + swap_halves(pc[0], lane);
}

// D_i = sum_j P_ij dP_ij over one 32-key block in accumulator layout (this
// lane's 16 keys of its query, then the other lane half's 16): D in the
// softmax-Jacobian form, from the fp32 weights and dP before any rounding.
// A row whose visible keys all lie in its first 32-key block takes this D in
// place of rowsum(dO o O): with the stored 16-bit O that sum carries O's
// rounding (relative 2^-9 for bf16), and with one or two keys dP - D is as
// small as that error, so dS, dQ and dK would inherit it at full size.
// Longer rows average it away.  Fixed order: r = 0..15, then the halves.
__device__ __forceinline__ float block_pdp_sum(const f32x16& p, const f32x16& dp, int lane) {
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s = fmaf(p[r], dp[r], s);
  return s + swap_halves(s, lane);
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (batch, head, 128-key tile).
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DkdvTile {
  static constexpr int NW = 4;
  static constexpr int BC = 32 * NW;  // keys per workgroup
  static constexpr int MB = (sizeof(T) == 4 && D >= 64) ? 1 : 2;
  static constexpr int BR = 32 * MB;  // query rows per iteration
  static constexpr int CH = Elt<T>::CH;
  static constexpr int EPW = 4 / sizeof(T);  // elements per 4-byte word
  // Q and dO tiles are read row-wise (S, dP) and through transpose reads
  // (dK, dV); bf16 transpose reads of a 32-column block touch columns up to
  // 31, so even a 16-wide tile gets rows of at least 32 elements.
  static constexpr int QS = lds_stride_words((D >= 32 ? D : 32) / EPW) * EPW;
  static constexpr int NB = D >= 32 ? D / 32 : 1;
  static constexpr int CMASK = (D >= 32 ? 32 : D) - 1;
  static constexpr int DCH = D / (2 * CH);
  static constexpr int CPB = 16 / CH;
  static constexpr int ROW_CH = D / CH;
  static constexpr int Q_CHUNKS = BR * ROW_CH;
  static constexpr int Q_PER_T = (Q_CHUNKS + 255) / 256;
  static constexpr int OCC = (D <= 64) ? 2 : 1;  // workgroups per CU the registers allow
};

// QP = 2 (fp32 grids too small to fill the device): the workgroup's 4 waves
// form 2 key groups of 32 keys (64 keys per workgroup), and the 2 waves of a
// group take alternate query steps (each iteration brings in two steps, one
// per wave), so the longest walk is halved without partial sums in memory;
// at the end the second wave of each group hands its dK, dV accumulators to
// the first through LDS.
template <typename T, int D, bool CAUSAL, int QP>
__global__ __launch_bounds__(256, (DkdvTile<T, D>::OCC)) void bwd_dkdv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, T* __restrict__ dK, T* __restrict__ dV, int Nmax,
    int BHkv, float sl2, float scale, int H, int G, const int* __restrict__ cu, int Ttot, int S,
    float* __restrict__ PartK, float* __restrict__ PartV, long long kv_rows, int snake) {
  using C = DkdvTile<T, D>;
  constexpr int CH = C::CH, BR = C::BR, MB = C::MB, QS = C::QS;
  constexpr int BC = C::BC / QP;  // keys per workgroup
  // Double-buffered query-side tiles (QP query steps each): one barrier per
  // iteration.
  __shared__ __attribute__((aligned(16))) T Qs[2][QP * BR * QS];
  __shared__ __attribute__((aligned(16))) T dOs[2][QP * BR * QS];
  __shared__ __attribute__((aligned(16))) float lse_s[2][QP * BR];
  __shared__ __attribute__((aligned(16))) float dl_s[2][QP * BR];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int kg = w % (C::NW / QP);  // key group (32 keys) of this wave
  const int qp = w / (C::NW / QP);  // which query step of each iteration it takes
  const int lin = blockIdx.x;
  // Key tile kt = 0 is the heaviest (causal); see causal_rank.
  const int kt = CAUSAL ? causal_rank(lin / (BHkv * S), (Nmax + BC - 1) / BC, snake != 0) : lin / (BHkv * S);
  const int sp = (lin % (BHkv * S)) / BHkv;  // which of the S pieces of the query-tile walk
  const int bhk = lin % BHkv;  // (sequence, key/value head); it serves query heads hk*G .. hk*G + G - 1
  const int bq = bhk / (H / G), hk = bhk % (H / G);
  const SeqRows skv = seq_rows(cu, Nmax, Ttot, bq, hk, H / G);
  const int N = skv.n;  // this sequence's length
  const size_t base = (size_t)skv.row0 * D;
  // Query-side pointers of the query head being walked (set per head below).
  const T* Qh = Q;
  const T* dOh = dO;
  const float* lseh = LSE;
  const float* dlh = Delta;
  const int kv0 = kt * BC;
  if (kv0 >= N) return;  // a tile past a shorter packed sequence
  const int kw = kv0 + 32 * kg;  // first key of this wave
  const int kj = kw + l32;       // key (accumulator column) owned by this lane

  // K and V rows of this lane as B operands of S = Q K^T and dP = dO V^T
  // (rows past N load row N-1; their weights are masked to 0).
  u32x4 kf[C::DCH], vf[C::DCH];
  {
    const size_t off = base + (size_t)min(kj, N - 1) * D + h * CH;
#pragma unroll
    for (int c = 0; c < C::DCH; ++c) {
      kf[c] = load16(K + off + c * 2 * CH);
      vf[c] = load16(V + off + c * 2 * CH);
    }
  }

  f32x16 dk[C::NB], dv[C::NB];
#pragma unroll
  for (int b = 0; b < C::NB; ++b) {
    dk[b] = f32x16{};
    dv[b] = f32x16{};
  }

  const int n_qt = (N + BR - 1) / BR;
  const int qt_first = CAUSAL ? kv0 / BR : 0;
  // This workgroup's piece of the walk: query tiles [qt_begin, qt_end).
  const int qt_begin = qt_first + (int)((long long)(n_qt - qt_first) * sp / S);
  const int qt_end = qt_first + (int)((long long)(n_qt - qt_first) * (sp + 1) / S);

  // The rows of QP consecutive query steps starting at step qt.
  constexpr int Q_CHUNKS = QP * C::Q_CHUNKS;
  constexpr int Q_PER_T = (Q_CHUNKS + 255) / 256;
  u32x4 qr[Q_PER_T], gr[Q_PER_T];
  float lr = 0.f, dr = 0.f;
  auto load_q = [&](int qt) {
#pragma unroll
    for (int u = 0; u < Q_PER_T; ++u) {
      const int c = tid + 256 * u;
      if (c < Q_CHUNKS) {
        const size_t off = (size_t)min(qt * BR + c / C::ROW_CH, N - 1) * D + (c % C::ROW_CH) * CH;
        qr[u] = load16(Qh + off);
        gr[u] = load16(dOh + off);
      }
    }
    if (tid < QP * BR) {
      const int i = qt * BR + tid;
      lr = i < N ? lseh[i] * kLog2e : INFINITY;  // rows past N get P = 0
      dr = i < N ? dlh[i] : 0.f;
    }
  };
  auto store_q = [&](int buf) {
#pragma unroll
    for (int u = 0; u < Q_PER_T; ++u) {
      const int c = tid + 256 * u;
      if (c < Q_CHUNKS) {
        const int row = c / C::ROW_CH, col = (c % C::ROW_CH) * CH;
        store16(&Qs[buf][row * QS + col], qr[u]);
        store16(&dOs[buf][row * QS + col], gr[u]);
      }
    }
    if (tid < QP * BR) {
      lse_s[buf][tid] = lr;
      dl_s[buf][tid] = dr;
    }
  };

  // A buffer is rewritten (store_q) one tile after its last reads, and every
  // wave has passed the barrier that follows those reads by then.
  const bool key_tail = kw + 31 >= N;  // this wave's keys reach past N
  // One 32-query block of a step, in three parts: the S and dP products, the
  // elementwise P = exp2(S*scale*log2e - LSE2), dS = P (dP - D) (rows past N
  // have LSE2 = +inf, so P = 0), and the dV^T += dO^T P, dK^T += Q^T dS
  // products, whose transposed operands are read straight from the
  // row-major tiles.
  auto mm_sdp = [&](const T* qs, const T* gs, int mb, f32x16& s, f32x16& dp) {
    s = f32x16{};
    dp = f32x16{};
    const T* qrow = qs + (32 * mb + l32) * QS + h * CH;
    const T* grow = gs + (32 * mb + l32) * QS + h * CH;
    if constexpr (sizeof(T) == 4) {
      // fp32: an MFMA chunk is four 64-cycle products, so fragments read
      // one chunk ahead hide the LDS latency and keep the registers for a
      // second wave per SIMD.
#pragma unroll
      for (int c = 0; c < C::DCH; ++c) {
        mfma_chunk<T>(s, load16(qrow + c * 2 * CH), kf[c]);
        mfma_chunk<T>(dp, load16(grow + c * 2 * CH), vf[c]);
      }
    } else {
    // All operand fragments first, so the wave waits on LDS once per phase.
    u32x4 qa[C::DCH], ga[C::DCH];
#pragma unroll
    for (int c = 0; c < C::DCH; ++c) {
      qa[c] = load16(qrow + c * 2 * CH);
      ga[c] = load16(grow + c * 2 * CH);
    }
#pragma unroll
    for (int c = 0; c < C::DCH; ++c) {
      mfma_chunk<T>(s, qa[c], kf[c]);
      mfma_chunk<T>(dp, ga[c], vf[c]);
    }
    }
  };
  auto grad = [&](const float* ls, const float* ds, int i0, int mb, f32x16& s, f32x16& dp, auto masked) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int il = 32 * mb + 8 * g + 4 * h;  // rows il..il+3 of this lane
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + il);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(ds + il);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * g + q;
        float p = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -l4[q]));
        if (decltype(masked)::value)  // bitwise, so it stays a select, not a branch
          p = ((CAUSAL & (kj > i0 + il + q)) | (kj >= N)) ? 0.f : p;
        s[r] = p;
        dp[r] = p * (dp[r] - d4[q]);
      }
    }
  };
  auto mm_kv = [&](const T* qs, const T* gs, int mb, const f32x16& s, const f32x16& dp) {
#pragma unroll
    for (int t = 0; t < C::CPB; ++t) {
      u32x4 ga[C::NB], qa[C::NB];
#pragma unroll
      for (int b = 0; b < C::NB; ++b) {
        ga[b] = load_rowcontract<T>(gs, QS, 32 * mb, t, 32 * b, C::CMASK, lane);
        qa[b] = load_rowcontract<T>(qs, QS, 32 * mb, t, 32 * b, C::CMASK, lane);
      }
      const u32x4 pb = pack_chunk<T>(s, t);
      const u32x4 sb = pack_chunk<T>(dp, t);
#pragma unroll
      for (int b = 0; b < C::NB; ++b) {
        mfma_chunk<T>(dv[b], ga[b], pb);
        mfma_chunk<T>(dk[b], qa[b], sb);
      }
    }
  };

  // Iteration it: query steps qt0 .. qt0 + QP - 1 in the buffers, this
  // wave's step qt = qt0 + qp.
  auto iteration = [&](int it, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const int buf = it & 1;
    const int qt0 = qt_begin + QP * it;
    const int qt = qt0 + qp;
    const T* qs = Qs[buf] + qp * BR * QS;
    const T* gs = dOs[buf] + qp * BR * QS;
    const float* ls = lse_s[buf] + qp * BR;
    const float* ds = dl_s[buf] + qp * BR;
    const int i0 = qt * BR;

    if (QP > 1 && qt >= qt_end) {
      // (the last iteration of an odd walk: this wave has no step)
    } else if (MASKED || MB != 2 || sizeof(T) != 2) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int ib = i0 + 32 * mb;
        if (kw < N && ib < N && (!CAUSAL || ib + 31 >= kw)) {
          f32x16 s, dp;
          mm_sdp(qs, gs, mb, s, dp);
          grad(ls, ds, i0, mb, s, dp, masked);
          mm_kv(qs, gs, mb, s, dp);
        }
      }
    } else {
      // Bulk step (every block live, no mask), ordered so the one wave per
      // SIMD has independent MFMAs issued ahead of each block's VALU work.
      // Blocks past N carry P = 0 (LSE2 = +inf) and need no test.
      f32x16 s0, dp0, s1, dp1;
      mm_sdp(qs, gs, 0, s0, dp0);
      mm_sdp(qs, gs, 1, s1, dp1);
      grad(ls, ds, i0, 0, s0, dp0, BoolC<false>{});
      mm_kv(qs, gs, 0, s0, dp0);
      grad(ls, ds, i0, 1, s1, dp1, BoolC<false>{});
      mm_kv(qs, gs, 1, s1, dp1);
    }
    if (qt0 + QP < qt_end) store_q(buf ^ 1);
    __syncthreads();
    if (qt0 + 2 * QP < qt_end) load_q(qt0 + 2 * QP);
  };
  // Query tiles that cross this key tile's diagonal band (or every tile when
  // the key tile is ragged) run with the mask; the rest need none.  The walk
  // is repeated for each query head that shares these keys (grouped-query
  // attention), accumulating into the same dK, dV.
  const int qt_mask_end = (kv0 + BC > N) ? n_qt : (CAUSAL ? min(n_qt, (kv0 + BC - 1) / BR + 1) : qt_begin);
  for (int g = 0; g < G; ++g) {
    const long long qrow0 = seq_rows(cu, Nmax, Ttot, bq, hk * G + g, H).row0;
    Qh = Q + (size_t)qrow0 * D;
    dOh = dO + (size_t)qrow0 * D;
    lseh = LSE + qrow0;
    dlh = Delta + qrow0;
    if (qt_begin < qt_end) {
      load_q(qt_begin);
      store_q(0);
      if (qt_begin + QP < qt_end) load_q(qt_begin + QP);
    }
    __syncthreads();
    if constexpr (QP == 1) {
      int qt = qt_begin, it = 0;
      for (; qt < min(qt_mask_end, qt_end); ++qt, ++it) iteration(it, BoolC<true>{});
      for (; qt < qt_end; ++qt, ++it) iteration(it, BoolC<false>{});
    } else {
      const int n_it = (qt_end - qt_begin + QP - 1) / QP;
      for (int it = 0; it < n_it; ++it) {
        if (qt_begin + QP * it + qp < qt_mask_end)  // uniform per wave
          iteration(it, BoolC<true>{});
        else
          iteration(it, BoolC<false>{});
      }
    }
  }

  if constexpr (QP > 1) {
    // The second wave of each key group leaves its accumulators in LDS (the
    // query tiles are no longer read), the first adds them to its own.
    constexpr int SLOT = 2 * C::NB * 16 * 64;  // floats per wave
    static_assert((C::NW / QP) * SLOT * sizeof(float) <= sizeof(Qs), "merge area");
    float* xm = reinterpret_cast<float*>(&Qs[0][0]) + kg * SLOT;
    __syncthreads();
    if (qp == 1) {
#pragma unroll
      for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          xm[(16 * b + r) * 64 + lane] = dk[b][r];
          xm[(16 * (C::NB + b) + r) * 64 + lane] = dv[b][r];
        }
    }
    __syncthreads();
    if (qp == 1) return;
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[b][r] += xm[(16 * b + r) * 64 + lane];
        dv[b][r] += xm[(16 * (C::NB + b) + r) * 64 + lane];
      }
  }

  if (S > 1) {
    // One of S partial sums over the query tiles: fp32 rows of [S][kv_rows,
    // d], dK already scaled (an empty piece writes zeros);
    // bwd_dkdv_reduce_kernel adds them up.
    if (kj < N) {
      const size_t row = (size_t)sp * kv_rows + skv.row0 + kj;
      float* pk = PartK + row * D;
      float* pv = PartV + row * D;
#pragma unroll
      for (int b = 0; b < C::NB; ++b) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * b + 8 * g + 4 * h;
          if (d0 < D) {
            *reinterpret_cast<f32x4*>(pk + d0) = f32x4{dk[b][4 * g] * scale, dk[b][4 * g + 1] * scale,
                                                        dk[b][4 * g + 2] * scale, dk[b][4 * g + 3] * scale};
            *reinterpret_cast<f32x4*>(pv + d0) = f32x4{dv[b][4 * g], dv[b][4 * g + 1], dv[b][4 * g + 2],
                                                        dv[b][4 * g + 3]};
          }
        }
      }
    }
    return;
  }

  if (kj < N) {
    T* dKj = dK + base + (size_t)kj * D;
    T* dVj = dV + base + (size_t)kj * D;
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * b + 8 * g + 4 * h;
        if (d0 < D) {
          store4<T>(dKj + d0, dk[b][4 * g] * scale, dk[b][4 * g + 1] * scale, dk[b][4 * g + 2] * scale,
                    dk[b][4 * g + 3] * scale);
          store4<T>(dVj + d0, dv[b][4 * g], dv[b][4 * g + 1], dv[b][4 * g + 2], dv[b][4 * g + 3]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (batch, head, 128-query tile).
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DqTile {
  static constexpr int NW = 4;
  static constexpr int BR = 32 * NW;                   // query rows per workgroup
  static constexpr int BC = sizeof(T) == 2 ? 64 : 32;  // keys per LDS tile
  static constexpr int CH = Elt<T>::CH;
  static constexpr int EPW = 4 / sizeof(T);
  // K is read row-wise (S^T) and through transpose reads (dQ^T); V only
  // row-wise (dP^T), which a 16-byte pad keeps conflict-free.
  static constexpr int KS = lds_stride_words((D >= 32 ? D : 32) / EPW) * EPW;
  static constexpr int VS = D + CH;
  static constexpr int NB = D >= 32 ? D / 32 : 1;
  static constexpr int CMASK = (D >= 32 ? 32 : D) - 1;
  static constexpr int DCH = D / (2 * CH);
  static constexpr int NJB = BC / 32;
  static constexpr int CPB = 16 / CH;
  static constexpr int ROW_CH = D / CH;
  static constexpr int CHUNKS = BC * ROW_CH;
  static constexpr int PER_T = (CHUNKS + 255) / 256;
  static constexpr int OCC = (sizeof(T) == 4 && D == 128) ? 1 : 2;  // workgroups per CU
};

// KP = 2 (fp32 grids too small to fill the device): the 4 waves form 2 row
// groups of 32 query rows (64 rows per workgroup), and the 2 waves of a
// group take alternate key tiles (each step brings in two tiles, one per
// wave), so the longest walk is halved without partial sums in memory; at
// the end the second wave of each group hands its dQ accumulators to the
// first through LDS.
template <typename T, int D, bool CAUSAL, int KP>
__global__ __launch_bounds__(256, (DqTile<T, D>::OCC)) void bwd_dq_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                        const T* __restrict__ V, const T* __restrict__ dO,
                                                        const T* __restrict__ O, const float* __restrict__ LSE,
                                                        float* __restrict__ Lse2, float* __restrict__ Delta,
                                                        T* __restrict__ dQ, int Nmax,
                                                        int BH, int num_qt, float sl2, float scale, int H, int G,
                                                        const int* __restrict__ cu, int Ttot, int S,
                                                        float* __restrict__ PartQ, long long rows, int snake) {
  using C = DqTile<T, D>;
  constexpr int CH = C::CH, BC = C::BC, KS = C::KS, VS = C::VS;
  constexpr int BR = C::BR / KP;  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) T Ks[2][KP * BC * KS];
  __shared__ __attribute__((aligned(16))) T Vs[2][KP * BC * VS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int qg = w % (C::NW / KP);  // row group (32 query rows) of this wave
  const int kp = w / (C::NW / KP);  // which key tile of each step it takes
  const int lin = blockIdx.x;
  const int qt = CAUSAL ? (num_qt - 1 - causal_rank(lin / (BH * S), num_qt, snake != 0)) : (lin / (BH * S));
  const int sp = (lin % (BH * S)) / BH;  // which of the S pieces of the key-tile walk
  const int bh = lin % BH;
  const SeqRows sq = seq_rows(cu, Nmax, Ttot, bh / H, bh % H, H);
  const int N = sq.n;  // this sequence's length
  const size_t base = (size_t)sq.row0 * D;
  const size_t kv_base = (size_t)seq_rows(cu, Nmax, Ttot, bh / H, (bh % H) / G, H / G).row0 * D;
  const T* Kh = K + kv_base;
  const T* Vh = V + kv_base;
  const int q0 = qt * BR;
  if (q0 >= N) return;  // a tile past a shorter packed sequence
  const int qw = q0 + 32 * qg;  // first query row of this wave
  const int qi = qw + l32;     // query row (column of S^T) owned by this lane

  // Q and dO rows of this lane (B operands); its LSE (base 2) and D, which
  // this kernel computes for its own rows and writes to the workspace for
  // the dK/dV kernel that runs after it.  Rows past N read row N-1 and are
  // never stored.
  const int qc = min(qi, N - 1);
  u32x4 qf[C::DCH], gf[C::DCH];
  float pc[C::DCH];
  {
    const size_t off = base + (size_t)qc * D + h * CH;
#pragma unroll
    for (int c = 0; c < C::DCH; ++c) {
      qf[c] = load16(Q + off + c * 2 * CH);
      gf[c] = load16(dO + off + c * 2 * CH);
    }
#pragma unroll
    for (int c = 0; c < C::DCH; ++c) pc[c] = dot_chunk<T>(load16(O + off + c * 2 * CH), gf[c]);
  }
  const float lse2 = LSE[sq.row0 + qc] * kLog2e;
  float dl = row_dot<C::DCH>(pc, lane);  // D = rowsum(dO * O)
  // Rows whose visible keys all lie in keys 0..31 take D = sum_j P_ij dP_ij
  // from that first 32-key block instead (block_pdp_sum).
  const bool d_from_block = (CAUSAL ? min(qi, N - 1) : N - 1) < 32;

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int n_kt = (kv_end + BC - 1) / BC;
  // This workgroup's piece of the walk: key tiles [kt_lo, kt_hi).  The one
  // piece that walks key tile 0 writes D and LSE * log2(e) of these rows
  // (with KP = 2, the wave of each pair that takes tile 0).
  const int kt_lo = (int)((long long)n_kt * sp / S);
  const int kt_hi = (int)((long long)n_kt * (sp + 1) / S);
  const bool writes_d = kt_lo == 0 && kt_lo < kt_hi && kp == 0;

  // The key and value rows of KP consecutive key tiles starting at tile kt.
  constexpr int CHUNKS = KP * C::CHUNKS;
  constexpr int PER_T = (CHUNKS + 255) / 256;
  u32x4 kr[PER_T], vr[PER_T];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int c = tid + 256 * u;
      if (c < CHUNKS) {
        const size_t off = (size_t)min(kt * BC + c / C::ROW_CH, N - 1) * D + (c % C::ROW_CH) * CH;
        kr[u] = load16(Kh + off);
        vr[u] = load16(Vh + off);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int c = tid + 256 * u;
      if (c < CHUNKS) {
        const int row = c / C::ROW_CH, col = (c % C::ROW_CH) * CH;
        store16(&Ks[buf][row * KS + col], kr[u]);
        store16(&Vs[buf][row * VS + col], vr[u]);
      }
    }
  };

  f32x16 dq[C::NB];
#pragma unroll
  for (int b = 0; b < C::NB; ++b) dq[b] = f32x16{};

  if (kt_lo < kt_hi) {
    load_tile(kt_lo);
    store_tile(0);
  }
  __syncthreads();

  // Step st: key tiles kt0 .. kt0 + KP - 1 in the buffers, this wave's tile
  // kt = kt0 + kp (none past kt_hi).
  auto tile = [&](int st, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const int kt0 = kt_lo + KP * st;
    const int kt = kt0 + kp;
    const bool more = kt0 + KP < kt_hi;
    if (more) load_tile(kt0 + KP);
    const T* ks = Ks[st & 1] + kp * BC * KS;
    const T* vs = Vs[st & 1] + kp * BC * VS;
    const int kb0 = kt * BC;
    const int last_key = CAUSAL ? min(qw + 31, N - 1) : N - 1;
    const int nlive = (KP > 1 && kt >= kt_hi) ? 0
                      : MASKED ? (last_key < kb0 ? 0 : min(C::NJB, (last_key - kb0) / 32 + 1)) : C::NJB;
#pragma unroll
    for (int jb = 0; jb < C::NJB; ++jb) {
      if (jb < nlive) {
        f32x16 s = f32x16{}, dp = f32x16{};
        const T* krow = ks + (32 * jb + l32) * KS + h * CH;
        const T* vrow = vs + (32 * jb + l32) * VS + h * CH;
#pragma unroll
        for (int c = 0; c < C::DCH; ++c) {
          mfma_chunk<T>(s, load16(krow + c * 2 * CH), qf[c]);
          mfma_chunk<T>(dp, load16(vrow + c * 2 * CH), gf[c]);
        }
        const int kb = kb0 + 32 * jb;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lse2));
          if (MASKED) {
            const int j = kb + acc_row(r, h);
            p = ((CAUSAL & (j > qi)) | (j >= N)) ? 0.f : p;  // a select, not a branch
          }
          s[r] = p;
        }
        if (kb == 0) {
          const float dx = block_pdp_sum(s, dp, lane);
          dl = d_from_block ? dx : dl;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = s[r] * (dp[r] - dl);
        // dQ^T += K^T dS^T: K^T through transpose reads of the key tile.
#pragma unroll
        for (int t = 0; t < C::CPB; ++t) {
          const u32x4 sb = pack_chunk<T>(dp, t);
#pragma unroll
          for (int b = 0; b < C::NB; ++b)
            mfma_chunk<T>(dq[b], load_rowcontract<T>(ks, KS, 32 * jb, t, 32 * b, C::CMASK, lane), sb);
        }
      }
    }
    if (more) store_tile((st + 1) & 1);
    __syncthreads();
  };
  // Key tiles wholly below every row of this query tile and wholly before N
  // need no mask; the diagonal and ragged tiles come last.
  const int kt_full = min(n_kt, CAUSAL ? min(q0, N) / BC : N / BC);
  if constexpr (KP == 1) {
    int kt = kt_lo;
    for (; kt < min(kt_full, kt_hi); ++kt) tile(kt - kt_lo, BoolC<false>{});
    for (; kt < kt_hi; ++kt) tile(kt - kt_lo, BoolC<true>{});
  } else {
    const int n_st = (kt_hi - kt_lo + KP - 1) / KP;
    for (int st = 0; st < n_st; ++st) {
      if (kt_lo + KP * st + kp < kt_full)  // uniform per wave
        tile(st, BoolC<false>{});
      else
        tile(st, BoolC<true>{});
    }
    // The second wave of each row group leaves its accumulators in LDS (the
    // tiles are no longer read), the first adds them to its own.
    constexpr int SLOT = C::NB * 16 * 64;  // floats per wave
    static_assert((C::NW / KP) * SLOT * sizeof(float) <= sizeof(Ks), "merge area");
    float* xm = reinterpret_cast<float*>(&Ks[0][0]) + qg * SLOT;
    __syncthreads();
    if (kp == 1) {
#pragma unroll
      for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) xm[(16 * b + r) * 64 + lane] = dq[b][r];
    }
    __syncthreads();
    if (kp == 1) return;
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[b][r] += xm[(16 * b + r) * 64 + lane];
  }
  if (writes_d && h == 0 && qi < N) {
    Delta[sq.row0 + qi] = dl;
    Lse2[sq.row0 + qi] = lse2;
  }

  if (S > 1) {
    // One of S partial sums over the key tiles, scaled, as fp32 rows of
    // [S][rows, d] (an empty piece writes zeros); bwd_dkdv_reduce_kernel adds
    // them up.
    if (qi < N) {
      float* pq = PartQ + ((size_t)sp * rows + sq.row0 + qi) * D;
#pragma unroll
      for (int b = 0; b < C::NB; ++b) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * b + 8 * g + 4 * h;
          if (d0 < D)
            *reinterpret_cast<f32x4*>(pq + d0) = f32x4{dq[b][4 * g] * scale, dq[b][4 * g + 1] * scale,
                                                        dq[b][4 * g + 2] * scale, dq[b][4 * g + 3] * scale};
        }
      }
    }
    return;
  }
  if (qi < N) {
    T* dQi = dQ + base + (size_t)qi * D;
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * b + 8 * g + 4 * h;
        if (d0 < D)
          store4<T>(dQi + d0, dq[b][4 * g] * scale, dq[b][4 * g + 1] * scale, dq[b][4 * g + 2] * scale,
                    dq[b][4 * g + 3] * scale);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV for the 16-bit types at d = 128: one 4-wave workgroup per (batch, head,
// 128-key tile), two workgroups per CU, so every SIMD runs two waves from
// different workgroups whose barriers are independent: one wave's softmax
// work can overlap the other's MFMAs without the two being held in step.
// Register budget (<= 256 per wave): K rows and the dK^T, dV^T accumulators
// stay in registers; V rows come from LDS.  Q and dO tiles (32 rows per
// step, double-buffered) are filled by direct global->LDS loads into
// unpadded 256-byte rows whose 16-byte chunks are XOR-swizzled (chunk c of
// row r at c ^ swz(r)): the 16 lanes reading one chunk of 16 consecutive
// rows, and the 32 lanes of a transpose read, both land on distinct banks.
// ---------------------------------------------------------------------------
namespace d128 {
constexpr int D = 128;
constexpr int ROWE = 128;  // elements per LDS row
constexpr int BC = 128;    // keys per workgroup
constexpr int BR = 32;     // query rows per step
constexpr int TILE_E = BR * ROWE;
using namespace fa2::tiles;
}  // namespace d128

// Each wave owns 32 keys; all four walk every 32-row query step.
template <typename T, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_d128_kernel(const T* __restrict__ Q,
                                                               const T* __restrict__ K,
                                                               const T* __restrict__ V,
                                                               const T* __restrict__ dO,
                                                               const float* __restrict__ Lse2,
                                                               const float* __restrict__ Delta,
                                                               T* __restrict__ dK, T* __restrict__ dV,
                                                               int Nmax, int BHkv, float sl2, float scale, int H,
                                                               int G, int S, float* __restrict__ PartK,
                                                               float* __restrict__ PartV, const int* __restrict__ cu,
                                                               int Ttot, long long kv_rows) {
  using namespace d128;
  constexpr int CH = 8, DCH = D / 16, NB = D / 32;
  __shared__ __attribute__((aligned(16))) T Vs[BC * ROWE];         // 32 KB
  __shared__ __attribute__((aligned(16))) T QdO[2][2][TILE_E];     // [buf][Q|dO], 32 KB
  __shared__ __attribute__((aligned(16))) float LD[2][64];         // [buf][LSE2 32 | D 32]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int lin = blockIdx.x;
  // Key tiles ascending: for causal the heaviest go first (causal_order
  // over the S * BHkv (piece, sequence, key/value head) triples).
  const CausalOrder co = CAUSAL ? causal_order(lin, BHkv * S, (Nmax + d128::BC - 1) / d128::BC, BHkv * S >= kHeadGroupedHeads)
                                : CausalOrder{lin / (BHkv * S), lin % (BHkv * S)};
  const int kt = co.rank;
  const int sp = co.head / BHkv;  // which 1/S of the group's query heads
  const int bhk = co.head % BHkv;  // (sequence, key/value head)
  const int gpw = G / S;       // query heads walked by this workgroup: h0 .. h0 + gpw - 1
  const int bq = bhk / (H / G), hk = bhk % (H / G);
  const int h0 = hk * G + sp * gpw;
  const SeqRows skv = seq_rows(cu, Nmax, Ttot, bq, hk, H / G);
  const int N = skv.n;  // this sequence's length
  const size_t base = (size_t)skv.row0 * D;
  if (kt * BC >= N) return;  // a tile past a shorter packed sequence
  const T* Vh = V + base;
  const int kv0 = kt * BC;
  const int kw = kv0 + 32 * w;  // first key of this wave
  const int kj = kw + l32;      // key owned by this lane
  // Query-side sources of the query head being walked (set per head below):
  // Q and dO as buffers, LSE * log2(e) and D.
  u32x4 rq, rdo;
  const float* lseh = Lse2;
  const float* dlh = Delta;

  u32x4 kf[DCH];
  {
    const T* krow = K + base + (size_t)min(kj, N - 1) * D + h * CH;
#pragma unroll
    for (int c = 0; c < DCH; ++c) kf[c] = load16(krow + c * 2 * CH);
  }
  f32x16 dk[NB], dv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    dk[b] = f32x16{};
    dv[b] = f32x16{};
  }

  const int n_qt = (N + BR - 1) / BR;
  const int qt_begin = CAUSAL ? kv0 / BR : 0;
  const int n_st = n_qt - qt_begin;  // >= 1

  // V tile: 32 one-kilobyte loads, 8 per wave (rows past N read row N-1).
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int k = 8 * w + u;
    const int r = 4 * k + (lane >> 4);
    const int c = (lane & 15) ^ swz(r);
    dload16(Vh + (size_t)min(kv0 + r, N - 1) * D + c * 8, &Vs[k * 512]);
  }
  // Q, dO, LSE2, D of step st into buffer buf: 2 tensors x 8 loads, 4 per
  // wave (waves 0-1 Q, 2-3 dO); wave 0 fetches LSE2 and D.  Complete steps
  // take the row offset as the uniform buffer offset; a ragged last step
  // clamps its rows to N-1 per lane.
  auto issue = [&](int st, int buf) {
    const int step = qt_begin + st;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = 4 * w + u;
      const int tens = q >> 3, k = q & 7;
      const int r = 4 * k + (lane >> 4);
      const int col = ((lane & 15) ^ swz(r)) * 16;
      const u32x4 rs = tens ? rdo : rq;
      if ((step + 1) * BR <= N)
        bload16(rs, r * 256 + col, step * BR * 256, &QdO[buf][tens][k * 512]);
      else
        bload16(rs, min(step * BR + r, N - 1) * 256 + col, 0, &QdO[buf][tens][k * 512]);
    }
    if (w == 0) {
      const int i = min(step * BR + l32, N - 1);
      dload4(h ? dlh + i : lseh + i, &LD[buf][0]);
    }
  };

  const SwzOffsets so = swz_offsets(lane);
  // One step: 32 query rows against this wave's 32 keys.
  auto step_body = [&](const T* qt, const T* gt, const float* ld, int i0, auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    // Launder the lane offsets so the per-fragment XORs are recomputed each
    // step instead of being hoisted into dozens of live registers.
    int rofs = so.rofs, tofs0 = so.tofs0, tofs1 = so.tofs1, kk = so.kk;
    asm volatile("" : "+v"(rofs), "+v"(tofs0), "+v"(tofs1), "+v"(kk));
    const char* vrow = reinterpret_cast<const char*>(Vs) + w * 32 * 256;
    f32x16 s = f32x16{}, dp = f32x16{};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      const int ro = rofs ^ (c << 5);
      mfma_chunk<T>(s, lds16(qt, ro), kf[c]);
      mfma_chunk<T>(dp, lds16(gt, ro), lds16(vrow, ro));
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int c = 0; c < DCH - 2; ++c) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
    const int t_causal = kj - i0 - 4 * h;  // masked when t_causal > c_r
    const int t_rows = N - i0 - 4 * h;     // masked when c_r >= t_rows
    const bool key_dead = kj >= N;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int il = 8 * g + 4 * h;  // rows il..il+3 of this lane
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(ld + il);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(ld + 32 + il);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * g + q;
        float p = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -l4[q]));
        if (MASKED) {
          const int c_r = 8 * g + q;
          p = ((CAUSAL & (t_causal > c_r)) | (c_r >= t_rows) | key_dead) ? 0.f : p;
        }
        s[r] = p;
        dp[r] = p * (dp[r] - d4[q]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pb = pack_chunk<T>(s, t);
      const u32x4 sb = pack_chunk<T>(dp, t);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int cb = ((b ^ kk) << 6) + t * 4096;
        mfma_chunk<T>(dv[b], tr_frag(gt, tofs0 + cb, tofs1 + cb), pb);
        mfma_chunk<T>(dk[b], tr_frag(qt, tofs0 + cb, tofs1 + cb), sb);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 13; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  auto step = [&](int st, auto masked) {
    const int buf = st & 1;
    if (st + 1 < n_st) issue(st + 1, buf ^ 1);
    const int i0 = (qt_begin + st) * BR;
    // Skip blocks with no visible key (all above the diagonal, or keys past
    // N); they would only add zeros.
    if (!decltype(masked)::value || (kw < N && (!CAUSAL || i0 + 31 >= kw)))
      step_body(QdO[buf][0], QdO[buf][1], LD[buf], i0, masked);
    wait_vmem();
    __syncthreads();
  };
  // Steps off the diagonal band, complete (32 rows < N) and on a complete key
  // tile need no mask; only a prefix (the diagonal) and the ragged end do.
  const int full_steps = N / BR - qt_begin;
  const int st_bulk_begin = (kv0 + BC > N) ? n_st : (CAUSAL ? min(n_st, BC / BR) : 0);
  const int st_bulk_end = max(st_bulk_begin, min(n_st, full_steps));
  // The walk is repeated for each query head that shares these keys
  // (grouped-query attention), accumulating into the same dK, dV.
  for (int g = 0; g < gpw; ++g) {
    const long long qrow0 = seq_rows(cu, Nmax, Ttot, bq, h0 + g, H).row0;
    rq = make_rsrc(Q + (size_t)qrow0 * D, (unsigned)N * D * 2);
    rdo = make_rsrc(dO + (size_t)qrow0 * D, (unsigned)N * D * 2);
    lseh = Lse2 + qrow0;
    dlh = Delta + qrow0;
    issue(0, 0);
    wait_vmem();
    __syncthreads();
    int st = 0;
    for (; st < st_bulk_begin; ++st) step(st, BoolC<true>{});
    if (st < st_bulk_end && (st & 1)) step(st++, BoolC<false>{});
    // Unmasked steps in pairs with literal buffers, so the LDS read bases
    // are immediates; the loads get the next buffer as an opaque scalar.
    for (; st + 2 <= st_bulk_end; st += 2) {
      int one, zero;
      asm volatile("s_mov_b32 %0, 1" : "=s"(one));
      asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
      issue(st + 1, one);
      step_body(QdO[0][0], QdO[0][1], LD[0], (qt_begin + st) * BR, BoolC<false>{});
      wait_vmem();
      __syncthreads();
      if (st + 2 < n_st) issue(st + 2, zero);
      step_body(QdO[1][0], QdO[1][1], LD[1], (qt_begin + st + 1) * BR, BoolC<false>{});
      wait_vmem();
      __syncthreads();
    }
    for (; st < st_bulk_end; ++st) step(st, BoolC<false>{});
    for (; st < n_st; ++st) step(st, BoolC<true>{});
  }

  if (S > 1) {
    // One of S partial sums over the group: fp32 rows of [S][kv_rows, d]
    // (kv_rows = the rows of dK), dK already scaled; bwd_dkdv_reduce_kernel
    // adds them up.
    if (kj < N) {
      const size_t row = (size_t)sp * kv_rows + skv.row0 + kj;
      float* pk = PartK + row * D;
      float* pv = PartV + row * D;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * b + 8 * g + 4 * h;
          *reinterpret_cast<f32x4*>(pk + d0) = f32x4{dk[b][4 * g] * scale, dk[b][4 * g + 1] * scale,
                                                      dk[b][4 * g + 2] * scale, dk[b][4 * g + 3] * scale};
          *reinterpret_cast<f32x4*>(pv + d0) = f32x4{dv[b][4 * g], dv[b][4 * g + 1], dv[b][4 * g + 2],
                                                      dv[b][4 * g + 3]};
        }
      }
    }
    return;
  }
  // Stage the bf16 results row-major in LDS (16-byte chunks swizzled like
  // the tiles): dK in the V tile, dV in the Q/dO buffers, both free now.
  T* sk = Vs;
  T* sv = &QdO[0][0][0];
  {
    const int row = 32 * w + l32;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int off = row * ROWE + (((4 * b + g) ^ swz(row)) << 3) + 4 * h;
        store4<T>(sk + off, dk[b][4 * g] * scale, dk[b][4 * g + 1] * scale, dk[b][4 * g + 2] * scale,
                  dk[b][4 * g + 3] * scale);
        store4<T>(sv + off, dv[b][4 * g], dv[b][4 * g + 1], dv[b][4 * g + 2], dv[b][4 * g + 3]);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 32 * w + 4 * i + (lane >> 4);
    const int ch = lane & 15;
    const int key = kv0 + row;
    if (key < N) {
      const int off = (row * ROWE + ((ch ^ swz(row)) << 3)) * 2;
      store16(dK + base + (size_t)key * D + ch * 8, lds16(sk, off));
      store16(dV + base + (size_t)key * D + ch * 8, lds16(sv, off));
    }
  }
}

// dK, dV for the 16-bit types at d = 64: the d = 128 kernel's pass with
// 128-byte LDS rows (chunk c of row r at c ^ swz64(r)), 8-row direct loads
// and half the accumulators.
namespace d64 {
constexpr int D = 64;
constexpr int ROWE = 64;   // elements per LDS row
constexpr int BC = 128;    // keys per workgroup
constexpr int BR = 32;     // query rows per step
constexpr int TILE_E = BR * ROWE;
using namespace fa2::tiles;
}  // namespace d64

// Three waves per SIMD without the mask (168 registers); the causal
// variant keeps two, where three would spill.
template <typename T, bool CAUSAL>
__global__ __launch_bounds__(256, CAUSAL ? 2 : 3) void bwd_dkdv_d64_kernel(const T* __restrict__ Q,
                                                               const T* __restrict__ K,
                                                               const T* __restrict__ V,
                                                               const T* __restrict__ dO,
                                                               const float* __restrict__ Lse2,
                                                               const float* __restrict__ Delta,
                                                               T* __restrict__ dK, T* __restrict__ dV,
                                                               int Nmax, int BHkv, float sl2, float scale, int H,
                                                               int G, int S, float* __restrict__ PartK,
                                                               float* __restrict__ PartV, const int* __restrict__ cu,
                                                               int Ttot, long long kv_rows) {
  using namespace d64;
  constexpr int CH = 8, DCH = D / 16, NB = D / 32;
  __shared__ __attribute__((aligned(16))) T Vs[BC * ROWE];         // 16 KB
  __shared__ __attribute__((aligned(16))) T QdO[2][2][TILE_E];     // [buf][Q|dO], 16 KB
  __shared__ __attribute__((aligned(16))) float LD[2][64];         // [buf][LSE2 32 | D 32]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int lin = blockIdx.x;
  // Key tiles ascending: for causal the heaviest go first (causal_order
  // over the S * BHkv (piece, sequence, key/value head) triples).
  const CausalOrder co = CAUSAL ? causal_order(lin, BHkv * S, (Nmax + d64::BC - 1) / d64::BC, BHkv * S >= kHeadGroupedHeads)
                                : CausalOrder{lin / (BHkv * S), lin % (BHkv * S)};
  const int kt = co.rank;
  const int sp = co.head / BHkv;  // which 1/S of the group's query heads
  const int bhk = co.head % BHkv;  // (sequence, key/value head)
  const int gpw = G / S;       // query heads walked by this workgroup: h0 .. h0 + gpw - 1
  const int bq = bhk / (H / G), hk = bhk % (H / G);
  const int h0 = hk * G + sp * gpw;
  const SeqRows skv = seq_rows(cu, Nmax, Ttot, bq, hk, H / G);
  const int N = skv.n;  // this sequence's length
  const size_t base = (size_t)skv.row0 * D;
  if (kt * BC >= N) return;  // a tile past a shorter packed sequence
  const T* Vh = V + base;
  const int kv0 = kt * BC;
  const int kw = kv0 + 32 * w;  // first key of this wave
  const int kj = kw + l32;      // key owned by this lane
  // Query-side sources of the query head being walked (set per head below):
  // Q and dO as buffers, LSE * log2(e) and D.
  u32x4 rq, rdo;
  const float* lseh = Lse2;
  const float* dlh = Delta;

  u32x4 kf[DCH];
  {
    const T* krow = K + base + (size_t)min(kj, N - 1) * D + h * CH;
#pragma unroll
    for (int c = 0; c < DCH; ++c) kf[c] = load16(krow + c * 2 * CH);
  }
  f32x16 dk[NB], dv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    dk[b] = f32x16{};
    dv[b] = f32x16{};
  }

  const int n_qt = (N + BR - 1) / BR;
  const int qt_begin = CAUSAL ? kv0 / BR : 0;
  const int n_st = n_qt - qt_begin;  // >= 1

  // V tile: 16 one-kilobyte loads of 8 rows, 4 per wave (rows past N read
  // row N-1).
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int k = 4 * w + u;
    const int r = 8 * k + (lane >> 3);
    const int c = (lane & 7) ^ swz64(r);
    dload16(Vh + (size_t)min(kv0 + r, N - 1) * D + c * 8, &Vs[k * 512]);
  }
  // Q, dO, LSE2, D of step st into buffer buf: 2 tensors x 4 loads of 8
  // rows, 2 per wave (waves 0-1 Q, 2-3 dO); wave 0 fetches LSE2 and D.
  // Complete steps take the row offset as the uniform buffer offset; a
  // ragged last step clamps its rows to N-1 per lane.
  auto issue = [&](int st, int buf) {
    const int step = qt_begin + st;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = 2 * w + u;
      const int tens = q >> 2, k = q & 3;
      const int r = 8 * k + (lane >> 3);
      const int col = ((lane & 7) ^ swz64(r)) * 16;
      const u32x4 rs = tens ? rdo : rq;
      if ((step + 1) * BR <= N)
        bload16(rs, r * 128 + col, step * BR * 128, &QdO[buf][tens][k * 512]);
      else
        bload16(rs, min(step * BR + r, N - 1) * 128 + col, 0, &QdO[buf][tens][k * 512]);
    }
    if (w == 0) {
      const int i = min(step * BR + l32, N - 1);
      dload4(h ? dlh + i : lseh + i, &LD[buf][0]);
    }
  };

  const SwzOffsets so = swz_offsets64(lane);
  // One step: 32 query rows against this wave's 32 keys.
  auto step_body = [&](const T* qt, const T* gt, const float* ld, int i0, auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    // Launder the lane offsets so the per-fragment XORs are recomputed each
    // step instead of being hoisted into dozens of live registers.
    int rofs = so.rofs, tofs0 = so.tofs0, tofs1 = so.tofs1, kk = so.kk;
    asm volatile("" : "+v"(rofs), "+v"(tofs0), "+v"(tofs1), "+v"(kk));
    const char* vrow = reinterpret_cast<const char*>(Vs) + w * 32 * 128;
    f32x16 s = f32x16{}, dp = f32x16{};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      const int ro = rofs ^ (c << 5);
      mfma_chunk<T>(s, lds16(qt, ro), kf[c]);
      mfma_chunk<T>(dp, lds16(gt, ro), lds16(vrow, ro));
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int c = 0; c < DCH - 2; ++c) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
    const int t_causal = kj - i0 - 4 * h;  // masked when t_causal > c_r
    const int t_rows = N - i0 - 4 * h;     // masked when c_r >= t_rows
    const bool key_dead = kj >= N;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int il = 8 * g + 4 * h;  // rows il..il+3 of this lane
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(ld + il);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(ld + 32 + il);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * g + q;
        float p = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -l4[q]));
        if (MASKED) {
          const int c_r = 8 * g + q;
          p = ((CAUSAL & (t_causal > c_r)) | (c_r >= t_rows) | key_dead) ? 0.f : p;
        }
        s[r] = p;
        dp[r] = p * (dp[r] - d4[q]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pb = pack_chunk<T>(s, t);
      const u32x4 sb = pack_chunk<T>(dp, t);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int cb = ((b ^ kk) << 6) + t * 2048;
        mfma_chunk<T>(dv[b], tr_frag(gt, tofs0 + cb, tofs1 + cb), pb);
        mfma_chunk<T>(dk[b], tr_frag(qt, tofs0 + cb, tofs1 + cb), sb);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  auto step = [&](int st, auto masked) {
    const int buf = st & 1;
    if (st + 1 < n_st) issue(st + 1, buf ^ 1);
    const int i0 = (qt_begin + st) * BR;
    // Skip blocks with no visible key (all above the diagonal, or keys past
    // N); they would only add zeros.
    if (!decltype(masked)::value || (kw < N && (!CAUSAL || i0 + 31 >= kw)))
      step_body(QdO[buf][0], QdO[buf][1], LD[buf], i0, masked);
    wait_vmem();
    __syncthreads();
  };
  // Steps off the diagonal band, complete (32 rows < N) and on a complete key
  // tile need no mask; only a prefix (the diagonal) and the ragged end do.
  const int full_steps = N / BR - qt_begin;
  const int st_bulk_begin = (kv0 + BC > N) ? n_st : (CAUSAL ? min(n_st, BC / BR) : 0);
  const int st_bulk_end = max(st_bulk_begin, min(n_st, full_steps));
  // The walk is repeated for each query head that shares these keys
  // (grouped-query attention), accumulating into the same dK, dV.
  for (int g = 0; g < gpw; ++g) {
    const long long qrow0 = seq_rows(cu, Nmax, Ttot, bq, h0 + g, H).row0;
    rq = make_rsrc(Q + (size_t)qrow0 * D, (unsigned)N * D * 2);
    rdo = make_rsrc(dO + (size_t)qrow0 * D, (unsigned)N * D * 2);
    lseh = Lse2 + qrow0;
    dlh = Delta + qrow0;
    issue(0, 0);
    wait_vmem();
    __syncthreads();
    int st = 0;
    for (; st < st_bulk_begin; ++st) step(st, BoolC<true>{});
    if (st < st_bulk_end && (st & 1)) step(st++, BoolC<false>{});
    // Unmasked steps in pairs with literal buffers, so the LDS read bases
    // are immediates; the loads get the next buffer as an opaque scalar.
    for (; st + 2 <= st_bulk_end; st += 2) {
      int one, zero;
      asm volatile("s_mov_b32 %0, 1" : "=s"(one));
      asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
      issue(st + 1, one);
      step_body(QdO[0][0], QdO[0][1], LD[0], (qt_begin + st) * BR, BoolC<false>{});
      wait_vmem();
      __syncthreads();
      if (st + 2 < n_st) issue(st + 2, zero);
      step_body(QdO[1][0], QdO[1][1], LD[1], (qt_begin + st + 1) * BR, BoolC<false>{});
      wait_vmem();
      __syncthreads();
    }
    for (; st < st_bulk_end; ++st) step(st, BoolC<false>{});
    for (; st < n_st; ++st) step(st, BoolC<true>{});
  }

  if (S > 1) {
    // One of S partial sums over the group: fp32 rows of [S][kv_rows, d]
    // (kv_rows = the rows of dK), dK already scaled; bwd_dkdv_reduce_kernel
    // adds them up.
    if (kj < N) {
      const size_t row = (size_t)sp * kv_rows + skv.row0 + kj;
      float* pk = PartK + row * D;
      float* pv = PartV + row * D;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * b + 8 * g + 4 * h;
          *reinterpret_cast<f32x4*>(pk + d0) = f32x4{dk[b][4 * g] * scale, dk[b][4 * g + 1] * scale,
                                                      dk[b][4 * g + 2] * scale, dk[b][4 * g + 3] * scale};
          *reinterpret_cast<f32x4*>(pv + d0) = f32x4{dv[b][4 * g], dv[b][4 * g + 1], dv[b][4 * g + 2],
                                                      dv[b][4 * g + 3]};
        }
      }
    }
    return;
  }
  // Stage the bf16 results row-major in LDS (16-byte chunks swizzled like
  // the tiles): dK in the V tile, dV in the Q/dO buffers, both free now.
  T* sk = Vs;
  T* sv = &QdO[0][0][0];
  {
    const int row = 32 * w + l32;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int off = row * ROWE + (((4 * b + g) ^ swz64(row)) << 3) + 4 * h;
        store4<T>(sk + off, dk[b][4 * g] * scale, dk[b][4 * g + 1] * scale, dk[b][4 * g + 2] * scale,
                  dk[b][4 * g + 3] * scale);
        store4<T>(sv + off, dv[b][4 * g], dv[b][4 * g + 1], dv[b][4 * g + 2], dv[b][4 * g + 3]);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * w + 8 * i + (lane >> 3);
    const int ch = lane & 7;
    const int key = kv0 + row;
    if (key < N) {
      const int off = (row * ROWE + ((ch ^ swz64(row)) << 3)) * 2;
      store16(dK + base + (size_t)key * D + ch * 8, lds16(sk, off));
      store16(dV + base + (size_t)key * D + ch * 8, lds16(sv, off));
    }
  }
}

// dQ for the 16-bit types at d = 128 and d = 64: the pass of bwd_dq_kernel
// organised like fwd_pp_kernel.  32-key blocks of K and V reach LDS through
// direct loads into a ring of 4 slots (unpadded swizzled rows: 256-byte rows
// swizzled by swz, 128-byte rows by swz64), issued 3 blocks ahead, one
// barrier per block; lane offsets of every fragment and load are computed
// once and the block loop is unrolled over the ring.
namespace dqpp {
// Workgroups per CU: at d = 64 three fit (3 x 32 KB of LDS).
constexpr int occupancy(int D) { return D == 64 ? 3 : 2; }
}  // namespace dqpp
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, dqpp::occupancy(D)) void bwd_dq_pp_kernel(const T* __restrict__ Q,
                                                              const T* __restrict__ K,
                                                              const T* __restrict__ V,
                                                              const T* __restrict__ dO,
                                                              const T* __restrict__ O,
                                                              const float* __restrict__ LSE,
                                                              float* __restrict__ Lse2,
                                                              float* __restrict__ Delta,
                                                              T* __restrict__ dQ, int Nmax, int BH, int num_qt,
                                                              float sl2, float scale, int H, int G,
                                                              const int* __restrict__ cu, int Ttot) {
  using namespace tiles;
  static_assert(D == 128 || D == 64, "bwd_dq_pp_kernel: d = 128 or 64");
  constexpr int KB = 32, BLK_E = KB * D, CH = 8, DCH = D / 16, NB = D / 32;
  constexpr int ROWB = 2 * D;       // bytes per LDS row
  constexpr int CPR = ROWB / 16;    // 16-byte chunks per row
  constexpr int RPL = 1024 / ROWB;  // rows per 1-KB wave load
  constexpr int LPT = KB / RPL;     // loads per tensor per block
  constexpr int LPW = 2 * LPT / 4;  // loads per wave per block
  constexpr int QB = 128;           // query rows per workgroup (4 waves x 32)
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
  const int q0 = qt * QB;
  if (q0 >= N) return;  // a tile past a shorter packed sequence
  const int qw = q0 + 32 * w;  // first query row of this wave
  const int qi = qw + l32;     // query row (column of S^T) owned by this lane
  // Waves 0-1 load K rows, waves 2-3 V rows: load u of wave w is number
  // q = LPW w + u, rows RPL (q % LPT) .. + RPL - 1 of the block.
  const long long kv_row0 = seq_rows(cu, Nmax, Ttot, bh / H, (bh % H) / G, H / G).row0;
  const u32x4 rsrc = make_rsrc((w < 2 ? K : V) + (size_t)kv_row0 * D, (unsigned)N * D * 2);
  T* const dst0 = w < 2 ? &Ks[0][0] : &Vs[0][0];

  const int kv_end = CAUSAL ? min(N, q0 + QB) : N;
  const int nb = (kv_end + KB - 1) / KB;

  // Per-lane constants: load offsets within a block and LDS fragment offsets
  // (row fragments by chunk, transpose fragments by column block and half).
  auto swz_row = [](int r) { return D == 128 ? swz(r) : swz64(r); };
  int voff[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int r = RPL * ((LPW * w + u) % LPT) + lane / CPR;
    voff[u] = r * ROWB + (((lane % CPR) ^ swz_row(r)) << 4);
  }
  const SwzOffsets so = D == 128 ? swz_offsets(lane) : swz_offsets64(lane);
  int kofs[DCH], tofs0[NB], tofs1[NB];
#pragma unroll
  for (int c = 0; c < DCH; ++c) kofs[c] = so.rofs ^ (c << 5);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    tofs0[b] = so.tofs0 + ((b ^ so.kk) << 6);
    tofs1[b] = so.tofs1 + ((b ^ so.kk) << 6);
  }
  // Block kb into slot (rows past N read row N-1; their keys are masked).
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

  // Q and dO rows of this lane (B operands), its LSE (base 2) and D, which
  // this kernel computes for its own rows and writes to the workspace for
  // the dK/dV kernel that runs after it.  Rows past N read row N-1 and are
  // never stored.
  const int qc = min(qi, N - 1);
  u32x4 qf[DCH], gf[DCH];
  float pc[DCH];
  {
    const size_t off = base + (size_t)qc * D + h * CH;
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      qf[c] = load16(Q + off + c * 2 * CH);
      gf[c] = load16(dO + off + c * 2 * CH);
    }
#pragma unroll
    for (int c = 0; c < DCH; ++c) pc[c] = dot_chunk<T>(load16(O + off + c * 2 * CH), gf[c]);
  }
  float dl = row_dot<DCH>(pc, lane);  // D = rowsum(dO * O)
  const float lse2 = LSE[sq.row0 + qc] * kLog2e;
  // Rows whose visible keys all lie in block 0 take D = sum_j P_ij dP_ij
  // from that block instead (block_pdp_sum); only the first query tile
  // (causal) or a sequence of at most 32 keys has such rows.
  const bool d_from_block = (CAUSAL ? min(qi, N - 1) : N - 1) < KB;
  const bool tile_has_block_d = CAUSAL ? q0 == 0 : N <= KB;
#pragma unroll
  for (int b = 0; b < PF; ++b)
    if (b < nb) issue(b, b);
  wait_vmem();
  __syncthreads();

  // S^T = K Q^T and dP^T = V dO^T for the block in slot.
  auto products = [&](int slot, f32x16& s, f32x16& dp) {
    s = f32x16{};
    dp = f32x16{};
    const char* kb_ = reinterpret_cast<const char*>(Ks[slot]);
    const char* vb_ = reinterpret_cast<const char*>(Vs[slot]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      mfma_chunk<T>(s, lds16(kb_, kofs[c]), qf[c]);
      mfma_chunk<T>(dp, lds16(vb_, kofs[c]), gf[c]);
    }
    // LDS reads run three chunks ahead of the products that use them.
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < DCH - 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x16 dq[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) dq[b] = f32x16{};

  // Block kb in slot SLOT: its products, dS^T = P^T (dP^T - D) and
  // dQ^T += K^T dS^T.  (The Q and dO rows and the dQ accumulators leave no
  // room for a second block's products in flight.)
  // FIRST: block 0 of a tile with d_from_block rows (it is always masked).
  auto block = [&](auto slotc, int kb, auto masked, auto first) {
    constexpr int SLOT = decltype(slotc)::value;
    constexpr bool MASKED = decltype(masked)::value;
    constexpr bool FIRST = decltype(first)::value;
    const bool ahead = kb + PF < nb;
    if (ahead) issue(kb + PF, (SLOT + PF) % R);
    f32x16 s, dp;
    products(SLOT, s, dp);
    const int k0 = kb * KB;
    if (FIRST) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lse2));
        const int j = acc_row(r, h);
        s[r] = ((CAUSAL & (j > qi)) | (j >= N)) ? 0.f : p;
      }
      const float dx = block_pdp_sum(s, dp, lane);
      dl = d_from_block ? dx : dl;
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = s[r] * (dp[r] - dl);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lse2));
        if (MASKED) {
          const int j = k0 + acc_row(r, h);
          p = ((CAUSAL & (j > qi)) | (j >= N)) ? 0.f : p;  // a select, not a branch
        }
        dp[r] = p * (dp[r] - dl);
      }
    }
    const char* kb_ = reinterpret_cast<const char*>(Ks[SLOT]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 sb = pack_chunk<T>(dp, t);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        mfma_chunk<T>(dq[b], tr_frag(kb_, tofs0[b] + t * 16 * ROWB, tofs1[b] + t * 16 * ROWB), sb);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 2 * NB - 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (ahead)
      wait_vmem_n<LPW>();
    else
      wait_vmem();
    __syncthreads();
  };
  // Blocks wholly below every row of this query tile and before N need no
  // mask; the diagonal and ragged blocks come last.
  const int nb_full = min(nb, CAUSAL ? min(q0, N) / KB : N / KB);
  int kb = 0;
  // (A tile with d_from_block rows has at most one full block, so its block 0
  // always runs in the loop below.)
  for (; kb + 4 <= nb_full; kb += 4) {
    block(IntC<0>{}, kb, BoolC<false>{}, BoolC<false>{});
    block(IntC<1>{}, kb + 1, BoolC<false>{}, BoolC<false>{});
    block(IntC<2>{}, kb + 2, BoolC<false>{}, BoolC<false>{});
    block(IntC<3>{}, kb + 3, BoolC<false>{}, BoolC<false>{});
  }
  for (; kb < nb; ++kb) {
    switch (kb & 3) {
      case 0:
        if (kb == 0 && tile_has_block_d)
          block(IntC<0>{}, kb, BoolC<true>{}, BoolC<true>{});
        else
          block(IntC<0>{}, kb, BoolC<true>{}, BoolC<false>{});
        break;
      case 1: block(IntC<1>{}, kb, BoolC<true>{}, BoolC<false>{}); break;
      case 2: block(IntC<2>{}, kb, BoolC<true>{}, BoolC<false>{}); break;
      default: block(IntC<3>{}, kb, BoolC<true>{}, BoolC<false>{}); break;
    }
  }
  if (h == 0 && qi < N) {
    Delta[sq.row0 + qi] = dl;
    Lse2[sq.row0 + qi] = lse2;
  }

  if (qi < N) {
    T* dQi = dQ + base + (size_t)qi * D;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * b + 8 * g + 4 * h;
        store4<T>(dQi + d0, dq[b][4 * g] * scale, dq[b][4 * g + 1] * scale, dq[b][4 * g + 2] * scale,
                  dq[b][4 * g + 3] * scale);
      }
    }
  }
}

// Sums of the S partial dK (blockIdx.y = 0) and dV (1) of a split
// grouped-query dK/dV stage, in the fixed order s = 0 .. S-1, rounded once
// to the output type: 4 elements per thread; n (elements per tensor) is a
// multiple of 4 since d is.  For a packed ragged batch (cu != null, rows of
// T per head, D elements per row) rows outside [cu[0], cu[B]) of a head
// belong to no sequence and are left alone.
template <typename T>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(const float* __restrict__ PartK,
                                                              const float* __restrict__ PartV, T* __restrict__ dK,
                                                              T* __restrict__ dV, long long n, int S,
                                                              const int* __restrict__ cu, int B, int Ttot, int D) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  if (cu != nullptr) {
    const int t = (int)((i / D) % Ttot);
    const int lo = min(max(cu[0], 0), Ttot), hi = min(max(cu[B], lo), Ttot);
    if (t < lo || t >= hi) return;
  }
  const float* Part = blockIdx.y ? PartV : PartK;
  T* Out = blockIdx.y ? dV : dK;
  f32x4 acc = *reinterpret_cast<const f32x4*>(Part + i);
  for (int sp = 1; sp < S; ++sp) acc += *reinterpret_cast<const f32x4*>(Part + (size_t)sp * n + i);
  store4<T>(Out + i, acc[0], acc[1], acc[2], acc[3]);
}

// Grids of at most this many workgroups (two per CU) take the snake order
// of causal_rank.
constexpr long long kSnakeGrid = 512;

template <typename T, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a, int stage) {
  const int BH = a.B * a.H;
  const int BHkv = a.B * a.Hkv;  // dK/dV workgroups run over key/value heads
  const int G = a.H / a.Hkv;     // query heads per key/value head
  // Rows of the key-side tensors: [B, Hkv, N], or [Hkv, T] for a packed
  // ragged batch.
  const long long kv_rows = a.cu ? (long long)a.Hkv * a.T : (long long)BHkv * a.N;
  const float sl2 = a.scale * kLog2e;
  // Stage 1 is the dQ kernel, which also computes D and LSE * log2(e) for
  // its rows; stage 2 the dK/dV kernel.
  if (stage == 1) {
    if constexpr (sizeof(T) == 2 && (D == 128 || D == 64)) {
      if (!force_generic_kernels()) {
        const int num_qt = (a.N + 127) / 128;
        const long long blocks = (long long)num_qt * BH;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((bwd_dq_pp_kernel<T, D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                           static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                           static_cast<const T*>(a.v), static_cast<const T*>(a.dO),
                           static_cast<const T*>(a.o), a.lse, a.lse2, a.delta, static_cast<T*>(a.dq), a.N, BH,
                           num_qt, sl2, a.scale, a.H, G, a.cu, a.T);
        return hipGetLastError();
      }
    }
    using C = DqTile<T, D>;
    // fp32 splits each query tile's key walk (a.dq_splits pieces, after the
    // paired walks of small grids).
    const int S = sizeof(T) == 4 ? a.dq_splits : 1;
    constexpr bool can_pair = sizeof(T) == 4 && D <= 64;
    const bool paired = can_pair && fp32_paired_walks(a.B, a.H, a.N, D, a.dtype);
    const int br = paired ? C::BR / 2 : C::BR;
    const int num_qt = (a.N + br - 1) / br;
    const long long blocks = (long long)num_qt * BH;
    if (blocks * S > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const long long rows = a.cu ? (long long)a.H * a.T : (long long)BH * a.N;
    if (paired)
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, can_pair ? 2 : 1>), dim3((unsigned)(blocks * S)), dim3(256), 0,
                         a.stream, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                         static_cast<const T*>(a.v), static_cast<const T*>(a.dO), static_cast<const T*>(a.o), a.lse,
                         a.lse2, a.delta, static_cast<T*>(a.dq), a.N, BH, num_qt, sl2, a.scale, a.H, G, a.cu, a.T, S,
                         a.part, rows, (int)(blocks * S <= kSnakeGrid));
    else
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, 1>), dim3((unsigned)(blocks * S)), dim3(256), 0, a.stream,
                         static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                         static_cast<const T*>(a.dO), static_cast<const T*>(a.o), a.lse, a.lse2, a.delta,
                         static_cast<T*>(a.dq), a.N, BH, num_qt, sl2, a.scale, a.H, G, a.cu, a.T, S, a.part, rows,
                         (int)(blocks * S <= kSnakeGrid));
    if (S > 1) {
      const long long n = rows * D;
      const unsigned rb = (unsigned)((n / 4 + 255) / 256);
      // (blockIdx.y = 0 only: the partial dQ sums into dq.)
      hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<T>), dim3(rb, 1), dim3(256), 0, a.stream, a.part, a.part,
                         static_cast<T*>(a.dq), static_cast<T*>(a.dq), n, S, a.cu, a.B, a.T, D);
    }
    return hipGetLastError();
  }
  if constexpr (sizeof(T) == 2 && D == 128) {
    // (The generic dK/dV kernel walks whole groups itself, so a forced
    // generic run never splits them and the partial sum does not run.)
    if (stage == 2 && !force_generic_kernels()) {
      const long long blocks = (long long)((a.N + d128::BC - 1) / d128::BC) * BHkv;
      if (blocks * a.splits > 0x7fffffffLL) return hipErrorInvalidConfiguration;
      const int S = a.splits;
      const long long n = kv_rows * D;  // elements of dK (and of dV)
      float* part_k = a.part;
      float* part_v = a.part + align256((size_t)S * n * sizeof(float)) / sizeof(float);
      hipLaunchKernelGGL((bwd_dkdv_d128_kernel<T, CAUSAL>), dim3((unsigned)(blocks * S)), dim3(256), 0, a.stream,
                         static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                         static_cast<const T*>(a.v), static_cast<const T*>(a.dO), a.lse2, a.delta,
                         static_cast<T*>(a.dk), static_cast<T*>(a.dv), a.N, BHkv, sl2, a.scale, a.H, G,
                         S, part_k, part_v, a.cu, a.T, kv_rows);
      if (S > 1) {
        const unsigned rb = (unsigned)((n / 4 + 255) / 256);
        hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<T>), dim3(rb, 2), dim3(256), 0, a.stream, part_k, part_v,
                           static_cast<T*>(a.dk), static_cast<T*>(a.dv), n, S, a.cu, a.B, a.T, D);
      }
      return hipGetLastError();
    }
  }
  if constexpr (sizeof(T) == 2 && D == 64) {
    if (stage == 2 && !force_generic_kernels()) {
      const long long blocks = (long long)((a.N + d64::BC - 1) / d64::BC) * BHkv;
      if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL((bwd_dkdv_d64_kernel<T, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                         static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                         static_cast<const T*>(a.dO), a.lse2, a.delta, static_cast<T*>(a.dk),
                         static_cast<T*>(a.dv), a.N, BHkv, sl2, a.scale, a.H, G, 1, a.part, a.part, a.cu, a.T,
                         kv_rows);
      return hipGetLastError();
    }
  }
  if (stage == 2) {
    using C = DkdvTile<T, D>;
    // fp32 splits each key tile's query walk (a.splits pieces, after the
    // paired walks of small grids); the 16-bit types walk it whole here
    // (their splits are the d = 128 kernel's).
    const int S = sizeof(T) == 4 ? a.splits : 1;
    constexpr bool can_pair = sizeof(T) == 4 && D <= 64;
    const bool paired = can_pair && fp32_paired_walks(a.B, a.Hkv, a.N, D, a.dtype);
    const int bc = paired ? C::BC / 2 : C::BC;
    const long long blocks = (long long)((a.N + bc - 1) / bc) * BHkv;
    if (blocks * S > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const long long n = kv_rows * D;  // elements of dK (and of dV)
    float* part_k = a.part;
    float* part_v = a.part + align256((size_t)S * n * sizeof(float)) / sizeof(float);
    if (paired)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, can_pair ? 2 : 1>), dim3((unsigned)(blocks * S)), dim3(256),
                         0, a.stream, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                         static_cast<const T*>(a.v), static_cast<const T*>(a.dO), a.lse, a.delta,
                         static_cast<T*>(a.dk), static_cast<T*>(a.dv), a.N, BHkv, sl2, a.scale, a.H, G, a.cu, a.T, S,
                         part_k, part_v, kv_rows, (int)(blocks * S <= kSnakeGrid));
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, 1>), dim3((unsigned)(blocks * S)), dim3(256), 0, a.stream,
                         static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                         static_cast<const T*>(a.dO), a.lse, a.delta, static_cast<T*>(a.dk), static_cast<T*>(a.dv),
                         a.N, BHkv, sl2, a.scale, a.H, G, a.cu, a.T, S, part_k, part_v, kv_rows,
                         (int)(blocks * S <= kSnakeGrid));
    if (S > 1) {
      const unsigned rb = (unsigned)((n / 4 + 255) / 256);
      hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<T>), dim3(rb, 2), dim3(256), 0, a.stream, part_k, part_v,
                         static_cast<T*>(a.dk), static_cast<T*>(a.dv), n, S, a.cu, a.B, a.T, D);
    }
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

template <typename T, bool CAUSAL>
static hipError_t launch_bwd_d(const BwdArgs& a, int stage) {
  switch (a.d) {
    case 16: return launch_bwd_t<T, 16, CAUSAL>(a, stage);
    case 32: return launch_bwd_t<T, 32, CAUSAL>(a, stage);
    case 64: return launch_bwd_t<T, 64, CAUSAL>(a, stage);
    case 128: return launch_bwd_t<T, 128, CAUSAL>(a, stage);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_backward_stage(const BwdArgs& a, int stage) {
  if (a.dtype == kBF16)
    return a.causal ? launch_bwd_d<__bf16, true>(a, stage) : launch_bwd_d<__bf16, false>(a, stage);
  if (a.dtype == kF16)
    return a.causal ? launch_bwd_d<_Float16, true>(a, stage) : launch_bwd_d<_Float16, false>(a, stage);
  return a.causal ? launch_bwd_d<float, true>(a, stage) : launch_bwd_d<float, false>(a, stage);
}

}  // namespace fa2
