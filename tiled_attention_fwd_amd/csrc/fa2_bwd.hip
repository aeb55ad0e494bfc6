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
//   bwd_pre_kernel   D = rowsum(dO o O) in fp32, and zeroing of the fp32 dQ
//                    accumulator (HBM-bound, one pass over O and dO).
//   bwd_kernel       one workgroup per (batch, head, 128-key tile); each of
//                    its 4 waves owns 32 keys and keeps K, V (as MFMA B
//                    operands) and its dK^T, dV^T accumulators in registers
//                    while it walks the query tiles.  Per query tile:
//                    S = Q K^T and dP = dO V^T on MFMA, P and dS in fp32,
//                    dV^T += dO^T P and dK^T += Q^T dS on MFMA (P and dS feed
//                    straight from the accumulator layout; Q and dO are also
//                    staged transposed in LDS), then dS goes through LDS and
//                    dQ_tile = dS K is computed on MFMA and added into the
//                    fp32 accumulator with atomics.
//   dq_convert_kernel  fp32 accumulator -> bf16 dQ (bf16 mode only).
// Causal: key tiles start at the first query tile that can see them and
// launch heaviest first; blocks entirely above the diagonal are skipped.
#include "fa2_common.hpp"
#include "fa2_launch.hpp"

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

// D_i = sum_k dO_ik O_ik; optionally zero row i of the fp32 dQ accumulator.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                      float* __restrict__ Delta, float* __restrict__ dQacc,
                                                      long long rows) {
  constexpr int CH = Elt<T>::CH;
  constexpr int TPR = D / CH;  // threads per row (2..32, a power of two)
  constexpr int RPB = 256 / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int cc = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    acc = dot_chunk<T>(load16(O + row * D + cc * CH), load16(dO + row * D + cc * CH));
    float* z = dQacc + row * D + cc * CH;
#pragma unroll
    for (int k = 0; k < CH / 4; ++k) store16(z + 4 * k, u32x4{0u, 0u, 0u, 0u});
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && cc == 0) Delta[row] = acc;
}

__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq,
                                                         long long n8) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long long)gridDim.x * 256) {
    const f32x4 lo = as_f32x4(load16(acc + 8 * i)), hi = as_f32x4(load16(acc + 8 * i + 4));
    const f32x2 p0 = {lo[0], lo[1]}, p1 = {lo[2], lo[3]}, p2 = {hi[0], hi[1]}, p3 = {hi[2], hi[3]};
    const u32x4 r = {__builtin_bit_cast(uint32_t, __builtin_convertvector(p0, bf16x2)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(p1, bf16x2)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(p2, bf16x2)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(p3, bf16x2))};
    store16(dq + 8 * i, r);
  }
}

template <typename T, int D>
struct BwdTile {
  static constexpr int NW = 4;
  static constexpr int BC = 32 * NW;  // keys per workgroup
  static constexpr int MB = (sizeof(T) == 4 && D == 128) ? 1 : 2;
  static constexpr int BR = 32 * MB;  // query rows per iteration
  static constexpr int CH = Elt<T>::CH;
  static constexpr int QS = D + CH;    // natural Q / dO tile row stride
  static constexpr int TS = BR + CH;   // transposed Q / dO tile row stride
  static constexpr int SS = BC + CH;   // dS tile row stride
  static constexpr int KTS = BC + CH;  // transposed K tile row stride
  static constexpr int NB = D >= 32 ? D / 32 : 1;
  static constexpr int DCH = D / (2 * CH);
  static constexpr int CPB = 16 / CH;
  static constexpr int ROW_CH = D / CH;
  static constexpr int T_UNITS = (BR / 4) * ROW_CH;
  static constexpr int T_PER_T = (T_UNITS + 255) / 256;
  static constexpr int K_UNITS = (BC / 4) * ROW_CH;
  static constexpr int K_PER_T = (K_UNITS + 255) / 256;
  static constexpr int SCH = BC / (2 * CH);  // chunks of the dQ contraction over keys
  static constexpr int NQB = MB * NB;        // 32x32 dQ output blocks per query tile
  static constexpr int QB_PER_W = (NQB + NW - 1) / NW;
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                     const T* __restrict__ V, const T* __restrict__ dO,
                                                     const float* __restrict__ LSE,
                                                     const float* __restrict__ Delta, float* __restrict__ dQacc,
                                                     T* __restrict__ dK, T* __restrict__ dV, int N, int BH,
                                                     float sl2, float scale) {
  using C = BwdTile<T, D>;
  constexpr int CH = C::CH, BR = C::BR, BC = C::BC, MB = C::MB;
  constexpr int QS = C::QS, TS = C::TS, SS = C::SS, KTS = C::KTS;
  __shared__ __attribute__((aligned(16))) T Qs[BR * QS];
  __shared__ __attribute__((aligned(16))) T dOs[BR * QS];
  __shared__ __attribute__((aligned(16))) T Qt[D * TS];
  __shared__ __attribute__((aligned(16))) T dOt[D * TS];
  __shared__ __attribute__((aligned(16))) T dSs[BR * SS];
  __shared__ __attribute__((aligned(16))) T Kt[D * KTS];
  __shared__ float lse_s[BR];
  __shared__ float dl_s[BR];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int lin = blockIdx.x;
  const int kt = lin / BH;  // ascending: for causal the heaviest key tiles go first
  const int bh = lin % BH;
  const size_t base = (size_t)bh * N * D;
  const T* Qh = Q + base;
  const T* Kh = K + base;
  const T* Vh = V + base;
  const T* dOh = dO + base;
  const float* lseh = LSE + (size_t)bh * N;
  const float* dlh = Delta + (size_t)bh * N;
  const int kv0 = kt * BC;
  const int kw = kv0 + 32 * w;  // first key of this wave
  const int kj = kw + l32;      // key (accumulator column) owned by this lane

  // K and V rows of this lane as B operands of S = Q K^T and dP = dO V^T.
  u32x4 kf[C::DCH], vf[C::DCH];
#pragma unroll
  for (int c = 0; c < C::DCH; ++c) {
    const int col = c * 2 * CH + h * CH;
    kf[c] = kj < N ? load16(Kh + (size_t)kj * D + col) : u32x4{0u, 0u, 0u, 0u};
    vf[c] = kj < N ? load16(Vh + (size_t)kj * D + col) : u32x4{0u, 0u, 0u, 0u};
  }
  // K tile transposed (d x keys, natural key order) for dQ = dS K.
#pragma unroll
  for (int u = 0; u < C::K_PER_T; ++u) {
    const int uu = tid + 256 * u;
    if (uu < C::K_UNITS) {
      const int j0 = kv0 + 4 * (uu / C::ROW_CH);
      const int col = (uu % C::ROW_CH) * CH;
      u32x4 r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r[e] = (j0 + e) < N ? load16(Kh + (size_t)(j0 + e) * D + col) : u32x4{0u, 0u, 0u, 0u};
      write_transposed4<T>(Kt, KTS, col, 4 * (uu / C::ROW_CH), r);
    }
  }

  f32x16 dk[C::NB], dv[C::NB];
#pragma unroll
  for (int b = 0; b < C::NB; ++b) {
    dk[b] = f32x16{};
    dv[b] = f32x16{};
  }

  const int n_qt = (N + BR - 1) / BR;
  const int qt_begin = CAUSAL ? kv0 / BR : 0;

  u32x4 qr[C::T_PER_T][4], gr[C::T_PER_T][4];
  float lr = 0.f, dr = 0.f;
  auto load_q = [&](int qt) {
#pragma unroll
    for (int s = 0; s < C::T_PER_T; ++s) {
      const int uu = tid + 256 * s;
      if (uu < C::T_UNITS) {
        const int i0 = qt * BR + 4 * (uu / C::ROW_CH);
        const int col = (uu % C::ROW_CH) * CH;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = (i0 + e) < N;
          qr[s][e] = ok ? load16(Qh + (size_t)(i0 + e) * D + col) : u32x4{0u, 0u, 0u, 0u};
          gr[s][e] = ok ? load16(dOh + (size_t)(i0 + e) * D + col) : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    if (tid < BR) {
      const int i = qt * BR + tid;
      lr = i < N ? lseh[i] * kLog2e : INFINITY;  // rows past N get P = 0
      dr = i < N ? dlh[i] : 0.f;
    }
  };
  auto store_q = [&]() {
#pragma unroll
    for (int s = 0; s < C::T_PER_T; ++s) {
      const int uu = tid + 256 * s;
      if (uu < C::T_UNITS) {
        const int rq = uu / C::ROW_CH;
        const int col = (uu % C::ROW_CH) * CH;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          store16(Qs + (4 * rq + e) * QS + col, qr[s][e]);
          store16(dOs + (4 * rq + e) * QS + col, gr[s][e]);
        }
        write_transposed4<T>(Qt, TS, col, swap_bits23(4 * rq), qr[s]);
        write_transposed4<T>(dOt, TS, col, swap_bits23(4 * rq), gr[s]);
      }
    }
    if (tid < BR) {
      lse_s[tid] = lr;
      dl_s[tid] = dr;
    }
  };

  if (qt_begin < n_qt) load_q(qt_begin);
  for (int qt = qt_begin; qt < n_qt; ++qt) {
    store_q();
    __syncthreads();
    if (qt + 1 < n_qt) load_q(qt + 1);
    const int i0 = qt * BR;

    f32x16 s[MB], dp[MB];
    bool live[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int ib = i0 + 32 * mb;
      live[mb] = kw < N && ib < N && (!CAUSAL || ib + 31 >= kw);
      if (live[mb]) {
        s[mb] = f32x16{};
        dp[mb] = f32x16{};
        const T* qrow = Qs + (32 * mb + l32) * QS + h * CH;
        const T* grow = dOs + (32 * mb + l32) * QS + h * CH;
#pragma unroll
        for (int c = 0; c < C::DCH; ++c) {
          mfma_chunk<T>(s[mb], load16(qrow + c * 2 * CH), kf[c]);
          mfma_chunk<T>(dp[mb], load16(grow + c * 2 * CH), vf[c]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int il = 32 * mb + acc_row(r, h);
          const int i = i0 + il;
          float p = __builtin_amdgcn_exp2f(fmaf(s[mb][r], sl2, -lse_s[il]));
          if ((CAUSAL && kj > i) || kj >= N) p = 0.f;
          s[mb][r] = p;
          dp[mb][r] = p * (dp[mb][r] - dl_s[il]);
        }
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS (contraction over the query rows).
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (live[mb]) {
#pragma unroll
        for (int t = 0; t < C::CPB; ++t) {
          const u32x4 pb = pack_chunk<T>(s[mb], t);
          const u32x4 sb = pack_chunk<T>(dp[mb], t);
          const int pos = 32 * mb + chunk_pos<CH>(t, h);
#pragma unroll
          for (int b = 0; b < C::NB; ++b) {
            const int trow = D >= 32 ? 32 * b + l32 : (l32 & (D - 1));
            mfma_chunk<T>(dv[b], load16(dOt + trow * TS + pos), pb);
            mfma_chunk<T>(dk[b], load16(Qt + trow * TS + pos), sb);
          }
        }
      }
    }
    // dS of this wave's 32 keys into the shared tile (zeros where skipped).
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dSs[(32 * mb + acc_row(r, h)) * SS + 32 * w + l32] = live[mb] ? from_f32<T>(dp[mb][r]) : from_f32<T>(0.f);
    }
    __syncthreads();
    // dQ_tile = dS (BR x BC) K (BC x D), added into the fp32 accumulator.
#pragma unroll
    for (int u = 0; u < C::QB_PER_W; ++u) {
      const int bidx = w + C::NW * u;
      if (bidx < C::NQB) {
        const int mb = bidx / C::NB, b = bidx % C::NB;
        const int ib = i0 + 32 * mb;
        if (ib < N && (!CAUSAL || ib + 31 >= kv0)) {
          f32x16 acc = f32x16{};
          const T* arow = dSs + (32 * mb + l32) * SS + h * CH;
          const T* brow = Kt + (D >= 32 ? 32 * b + l32 : (l32 & (D - 1))) * KTS + h * CH;
#pragma unroll
          for (int c = 0; c < C::SCH; ++c) mfma_chunk<T>(acc, load16(arow + c * 2 * CH), load16(brow + c * 2 * CH));
          const int dcol = 32 * b + l32;
          if (dcol < D) {
            float* dst = dQacc + base + dcol;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int i = ib + acc_row(r, h);
              if (i < N) unsafeAtomicAdd(dst + (size_t)i * D, acc[r] * scale);
            }
          }
        }
      }
    }
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

template <typename T, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a, int stage) {
  using C = BwdTile<T, D>;
  const int BH = a.B * a.H;
  const long long rows = (long long)BH * a.N;
  if (stage == 1) {
    constexpr int RPB = 256 / (D / Elt<T>::CH);
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       a.stream, static_cast<const T*>(a.o), static_cast<const T*>(a.dO), a.delta, a.dq_acc,
                       rows);
    return hipGetLastError();
  }
  if (stage == 2) {
    const long long blocks = (long long)((a.N + C::BC - 1) / C::BC) * BH;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_kernel<T, D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       static_cast<const T*>(a.dO), a.lse, a.delta, a.dq_acc, static_cast<T*>(a.dk),
                       static_cast<T*>(a.dv), a.N, BH, a.scale * kLog2e, a.scale);
    return hipGetLastError();
  }
  if (stage == 3) {
    if (a.dtype != kBF16) return hipSuccess;  // fp32 mode accumulates into dq directly
    const long long n8 = rows * D / 8;
    long long g = (n8 + 255) / 256;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)g), dim3(256), 0, a.stream, a.dq_acc,
                       static_cast<__bf16*>(a.dq), n8);
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
  return a.causal ? launch_bwd_d<float, true>(a, stage) : launch_bwd_d<float, false>(a, stage);
}

}  // namespace fa2
