// fa2_decode.hip -- flash-decoding: a few new queries against a long key/value
// cache, bf16 or fp16, d = 128 or 64.
//
// The article "Revolutionizing Web-Based AI: How a Plain JavaScript Prototype
// Paved the Way for High-Performance WebGPU Flash Attention 2" names
// flash-decoding as a next primitive (section "Next Frontiers in WebGPU ML",
// "Broader Opset Support").  It computes the same softmax attention as the
// forward pass, for N_q queries that sit at the last N_q positions of a
// sequence of N_k keys (causal: query i keeps keys j <= N_k - N_q + i).
//
// With N_q small there are too few query rows to spread over the device, so
// the cache is split instead: workgroup (b, key/value head, split, row block)
// walks one chunk of the cache for up to 32 query rows and keeps a running
// max, running sum and unnormalised output like the forward pass; a second
// kernel merges the chunks' normalised outputs with weights exp(LSE_s - max)
// (the rescaling of the online softmax applied once more).  The rows of a
// workgroup are the G query heads of one key/value head times the N_q
// queries, packed into the 32 columns of the score product, so a grouped
// cache is read once for its whole group.
//
// The pass reads the cache once: 2 N_k d s bytes per key/value head against
// about 4 N_k d flops per row, a few flops per byte, so it is bound by HBM.
// The kernel is built for bytes in flight: one wave per workgroup with its
// own 4-slot ring of 32-key K and V blocks (64 KB of LDS at d = 128, two
// workgroups per CU; 32 KB at d = 64), three blocks loaded ahead by direct global-to-LDS loads, and no
// barrier at all (a wave only reads what it loaded itself, after its own
// vmcnt wait).  The products use the forward's layout: S^T = K Q^T so the
// lane owning a row keeps m and l as scalars, and P is the B operand of
// O^T += V^T P^T with V^T read by transposed LDS loads.
#include "fa2_launch.hpp"
#include "fa2_swz.hpp"

namespace fa2 {
namespace {

namespace dec {
constexpr int KB = 32;           // keys per block
constexpr int R = 4, PF = R - 1; // ring slots, blocks loaded ahead
// 1-KB direct loads per K (or V) block: 8 at d = 128, 4 at d = 64.
constexpr int loads(int D) { return KB * D * 2 / 1024; }
static_assert(PF >= 1 && PF <= 3, "the waits below are written out for up to 3 blocks ahead");
}  // namespace dec

// s_waitcnt vmcnt(2 L n), expcnt and lgkmcnt at their maxima: all but the
// last n blocks' loads (2 x L per block, L = dec::loads(D)) done.  vmcnt's
// low four bits sit in bits 3:0 of the immediate, its high two in bits
// 15:14.  The empty asm keeps the compiler from moving LDS reads above the
// wait.
template <int D, int NBLK>
__device__ __forceinline__ void wait_blocks() {
  constexpr int c = 2 * dec::loads(D) * NBLK;
  static_assert(c < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((c & 15) | ((c >> 4) << 14) | 0x0F70);
  asm volatile("" ::: "memory");
}

// One wave: rows rb*32 .. rb*32+31 of the M = G * N_q rows of key/value head
// bhk = b * Hkv + kv, keys of blocks [sp*cb, min(nbk, (sp+1)*cb)).  Row r is
// query head kv*G + r / N_q, query r % N_q.  With S == 1 the wave writes O
// and LSE; otherwise its normalised O rows (fp32) and base-2 LSE go to
// PartO[sp], PartL[sp] (LSE = -inf and O = 0 for a row that sees no key of
// the chunk).
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(64) void decode_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                    const T* __restrict__ V, T* __restrict__ O,
                                                    float* __restrict__ LSE, float* __restrict__ PartO,
                                                    float* __restrict__ PartL, int Nq, int Nk, int H, int G,
                                                    int Hkv, int n_rb, int S, int cb, long long rows,
                                                    float sl2) {
  using namespace tiles;
  static_assert(D == 128 || D == 64, "decode_kernel: d = 128 or 64");
  constexpr int KB = dec::KB, BLK_E = KB * D, R = dec::R, PF = dec::PF, LOADS = dec::loads(D);
  constexpr int CH = 8, DCH = D / 16, NB = D / 32;
  constexpr int ROWB = 2 * D;       // bytes per LDS row
  constexpr int CPR = ROWB / 16;    // 16-byte chunks per row
  constexpr int RPL = 1024 / ROWB;  // rows per 1-KB load
  constexpr int LPP = 16 / RPL;     // loads per 16 rows (the swizzles' period)
  __shared__ __attribute__((aligned(16))) T Ks[R][BLK_E];
  __shared__ __attribute__((aligned(16))) T Vs[R][BLK_E];

  const int lane = threadIdx.x;
  const int l32 = lane & 31, h = lane >> 5;
  const int lin = blockIdx.x;
  const int rb = lin % n_rb;
  const int sp = (lin / n_rb) % S;
  const int bhk = lin / (n_rb * S);
  const int b = bhk / Hkv, kv = bhk % Hkv;
  const int M = G * Nq;
  const bool row_live = rb * 32 + l32 < M;
  const int r = min(rb * 32 + l32, M - 1);  // padding rows repeat the last row
  const int gq = r / Nq, qi = r % Nq;
  const long long row = ((long long)b * H + (long long)kv * G + gq) * Nq + qi;  // in [B, H, N_q]
  const int last = CAUSAL ? qi + (Nk - Nq) : Nk - 1;  // last key this row sees

  const size_t kv_base = (size_t)bhk * Nk * D;
  const u32x4 rk = make_rsrc(K + kv_base, (unsigned)Nk * D * 2);
  const u32x4 rv = make_rsrc(V + kv_base, (unsigned)Nk * D * 2);
  const int nbk = (Nk + KB - 1) / KB;
  const int kb0 = sp * cb;
  const int nb = min(nbk, kb0 + cb) - kb0;  // >= 1: the host leaves no split empty

  // Direct loads: load u of a block brings rows RPL u .. RPL u + RPL - 1
  // (1 KB) into bytes u*1024 .. of the slot; voff[u % LPP] + (u / LPP) *
  // 16 ROWB is the lane's byte offset in the block (swizzled chunk, as the
  // LDS tile wants; both swizzles repeat every 16 rows).
  auto swz_row = [](int r) { return D == 128 ? swz(r) : swz64(r); };
  int voff[LPP];
#pragma unroll
  for (int u = 0; u < LPP; ++u) {
    const int rr = RPL * u + lane / CPR;
    voff[u] = rr * ROWB + (((lane % CPR) ^ swz_row(rr)) << 4);
  }
  const SwzOffsets so = D == 128 ? swz_offsets(lane) : swz_offsets64(lane);
  int kofs[DCH], vofs0[NB], vofs1[NB];
#pragma unroll
  for (int c = 0; c < DCH; ++c) kofs[c] = so.rofs ^ (c << 5);
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    vofs0[bb] = so.tofs0 + ((bb ^ so.kk) << 6);
    vofs1[bb] = so.tofs1 + ((bb ^ so.kk) << 6);
  }

  // Block kb into slot (rows past N_k read row N_k - 1; they are masked).
  auto issue = [&](int kb, int slot) {
    const int row0 = kb * KB;
    T* dk = &Ks[slot][0];
    T* dv = &Vs[slot][0];
    if (row0 + KB <= Nk) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u)
        bload16(rk, voff[u % LPP] + (u / LPP) * 16 * ROWB, row0 * ROWB, dk + u * 512);
#pragma unroll
      for (int u = 0; u < LOADS; ++u)
        bload16(rv, voff[u % LPP] + (u / LPP) * 16 * ROWB, row0 * ROWB, dv + u * 512);
    } else {
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int rr = RPL * u + lane / CPR;
        const int off = min(row0 + rr, Nk - 1) * ROWB + (voff[u % LPP] & (ROWB - 1));
        bload16(rk, off, 0, dk + u * 512);
        bload16(rv, off, 0, dv + u * 512);
      }
    }
  };

  u32x4 qf[DCH];
  {
    const T* qrow = Q + row * D + h * CH;
#pragma unroll
    for (int c = 0; c < DCH; ++c) qf[c] = load16(qrow + c * 2 * CH);
  }
  negate_fragments_if<T>(qf, DCH, sl2);
#pragma unroll
  for (int t = 0; t < PF; ++t)
    if (t < nb) issue(kb0 + t, t);

  f32x16 o[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) o[bb] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled logits, base-2 units
  float l_run = 0.f;        // this lane half's share of the running sum

  // Block t of the chunk, in ring slot SLOT = t % R.
  auto block = [&](auto slotc, int t, auto masked) {
    constexpr int SLOT = decltype(slotc)::value;
    constexpr bool MASKED = decltype(masked)::value;
    const int ahead = nb - 1 - t;  // blocks of the chunk after this one
    if (ahead >= PF) {
      issue(kb0 + t + PF, (SLOT + PF) % R);  // that slot held block t - 1, already consumed
      wait_blocks<D, PF>();
    } else if (ahead == 2) {
      wait_blocks<D, 2>();
    } else if (ahead == 1) {
      wait_blocks<D, 1>();
    } else {
      wait_blocks<D, 0>();
    }
    f32x16 s = f32x16{};
    {
      const char* kb_ = reinterpret_cast<const char*>(Ks[SLOT]);
#pragma unroll
      for (int c = 0; c < DCH; ++c) mfma_chunk<T>(s, lds16(kb_, kofs[c]), qf[c]);
    }
    if (MASKED) {
      const int k0 = (kb0 + t) * KB;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = (k0 + acc_row(i, h) > last) ? -INFINITY : s[i];
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, swap_halves(mx, lane));
    const float m_cand = mx * sl2;
    const bool grow = m_cand > m_run + kSlack;
    if (__builtin_expect(__any(grow), 0)) {
      asm volatile("");
      const float m_new = grow ? m_cand : m_run;
      const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) o[bb] *= alpha;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    float l_blk = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, neg_m));
      l_blk += s[i];
    }
    l_run += l_blk;
    const char* vb_ = reinterpret_cast<const char*>(Vs[SLOT]);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const u32x4 pb = pack_chunk<T>(s, tt);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
        mfma_chunk<T>(o[bb], tr_frag(vb_, vofs0[bb] + tt * 16 * ROWB, vofs1[bb] + tt * 16 * ROWB), pb);
    }
  };

  // Blocks whose every key is visible to every row (below the first row's
  // diagonal, before N_k) need no mask.
  const int full_end = (CAUSAL ? Nk - Nq + 1 : Nk) / KB;
  const int t_full = max(0, min(nb, full_end - kb0));
  int t = 0;
  // Unmasked blocks R at a time, slot I of the ring for block t + I.
  auto bulk = [&](auto self, auto ic) {
    constexpr int I = decltype(ic)::value;
    if constexpr (I < R) {
      block(IntC<I>{}, t + I, BoolC<false>{});
      self(self, IntC<I + 1>{});
    }
  };
  for (; t + R <= t_full; t += R) bulk(bulk, IntC<0>{});
  // The rest one at a time, the slot picked at run time among R bodies.
  auto one = [&](auto self, auto ic) {
    constexpr int I = decltype(ic)::value;
    if constexpr (I < R) {
      if (t % R == I)
        block(IntC<I>{}, t, BoolC<true>{});
      else
        self(self, IntC<I + 1>{});
    }
  };
  for (; t < nb; ++t) one(one, IntC<0>{});

  const float l_tot = l_run + swap_halves(l_run, lane);
  if (!row_live) return;
  if (S == 1) {
    // The whole cache: every row sees key 0, so l_tot > 0.
    const float inv = 1.0f / l_tot;
    T* Oi = O + row * D;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * bb + 8 * g + 4 * h;
        store4<T>(Oi + d0, o[bb][4 * g] * inv, o[bb][4 * g + 1] * inv, o[bb][4 * g + 2] * inv,
                  o[bb][4 * g + 3] * inv);
      }
    }
    if (h == 0) LSE[row] = (m_run + log2f(l_tot)) * kLn2;
    return;
  }
  const bool empty = l_tot == 0.f;
  const float inv = empty ? 0.f : 1.0f / l_tot;
  float* po = PartO + ((size_t)sp * rows + row) * D;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * bb + 8 * g + 4 * h;
      *reinterpret_cast<f32x4*>(po + d0) =
          f32x4{o[bb][4 * g] * inv, o[bb][4 * g + 1] * inv, o[bb][4 * g + 2] * inv, o[bb][4 * g + 3] * inv};
    }
  }
  if (h == 0) PartL[(size_t)sp * rows + row] = empty ? -INFINITY : m_run + log2f(l_tot);
}

// Merge of the S chunks of each row: with L_s the chunks' base-2 LSE and
// L* = max_s L_s, w_s = 2^(L_s - L*), O = sum_s w_s O_s / sum_s w_s and
// LSE = (L* + log2 sum_s w_s) ln 2.  D / 4 threads per row, 4 elements each;
// every row has at least one chunk with a visible key, so L* is finite.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ PartO,
                                                           const float* __restrict__ PartL, T* __restrict__ O,
                                                           float* __restrict__ LSE, long long rows, int S) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = idx / (D / 4);
  const int c = (int)(idx % (D / 4)) * 4;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, PartL[(size_t)s * rows + row]);
  float wsum = 0.f;
  f32x4 acc = f32x4{};
  for (int s = 0; s < S; ++s) {
    const float w = exp2f(PartL[(size_t)s * rows + row] - mx);
    wsum += w;
    acc += w * *reinterpret_cast<const f32x4*>(PartO + ((size_t)s * rows + row) * D + c);
  }
  const float inv = 1.0f / wsum;
  store4<T>(O + row * D + c, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  if (c == 0) LSE[row] = (mx + log2f(wsum)) * kLn2;
}

}  // namespace

template <typename T, int D>
static hipError_t launch_decode_t(const DecArgs& a) {
  const DecodePlan p = decode_plan(a.B, a.H, a.Hkv, a.Nq, a.Nk);
  const long long rows = (long long)a.B * a.H * a.Nq;
  const long long blocks = (long long)a.B * a.Hkv * p.splits * p.row_blocks;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  float* part_o = a.workspace;
  float* part_l = a.workspace + align256((size_t)p.splits * rows * D * sizeof(float)) / sizeof(float);
  const float sl2 = a.scale * kLog2e;
  const int G = a.H / a.Hkv;
  if (a.causal)
    hipLaunchKernelGGL((decode_kernel<T, D, true>), dim3((unsigned)blocks), dim3(64), 0, a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       static_cast<T*>(a.o), a.lse, part_o, part_l, a.Nq, a.Nk, a.H, G, a.Hkv, p.row_blocks,
                       p.splits, p.chunk_blocks, rows, sl2);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, false>), dim3((unsigned)blocks), dim3(64), 0, a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       static_cast<T*>(a.o), a.lse, part_o, part_l, a.Nq, a.Nk, a.H, G, a.Hkv, p.row_blocks,
                       p.splits, p.chunk_blocks, rows, sl2);
  if (p.splits > 1) {
    const long long threads = rows * (D / 4);
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, a.stream,
                       part_o, part_l, static_cast<T*>(a.o), a.lse, rows, p.splits);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a) {
  if (a.d == 64) return a.dtype == kF16 ? launch_decode_t<_Float16, 64>(a) : launch_decode_t<__bf16, 64>(a);
  if (a.d == 128) return a.dtype == kF16 ? launch_decode_t<_Float16, 128>(a) : launch_decode_t<__bf16, 128>(a);
  return hipErrorInvalidValue;
}

}  // namespace fa2
