// Chunked parallel prefill of the gated delta rule (gfx950), fp32 inputs.
//
// This is the full-precision path: every matrix product runs on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32), so it keeps the result within
// fp32 rounding of the exact recurrence. The bf16-input path, which is the
// one tuned for throughput, lives in chunk_fwd.hip.
//
// The recurrence (page "NLP——技术报告解读-Qwen3.8-Flash-Next", section
// "Gated DeltaNet 核心机制") is evaluated 64 tokens at a time. Inside a chunk
// that starts from state S, with g_r the in-chunk running sum of log alpha,
// gamma_r = exp(g_r), G_ri = exp(g_r - g_i) for r >= i, and E the matrix of
// beta-scaled prediction errors, unrolling the erase-write rule gives
//     (I + A) E = diag(beta) (V - diag(gamma) K S),
//     A = strictly_lower(diag(beta) (K K^T o G))
//     Y = diag(gamma) Q S + tril(Q K^T o G) E
//     S <- gamma_C S + Kt^T E,     Kt_r = exp(g_C - g_r) k_r,
// so each chunk needs the unit-lower-triangular inverse T = (I + A)^{-1}
// (the UT transform of the compact WY representation), and the rest is dense
// products. Only exponentials of non-positive numbers are formed.
//
// One workgroup owns one (sequence, head, DVT-column tile of S) and walks its
// chunks in order; the fp32 state stays in registers for the whole sequence.
// Each wave owns a 16-column slab of the tile. Per chunk:
//   1. every wave scans the 64 gates (wavefront prefix sum), the workgroup
//      stages K, Q (and Kt^T, V) in LDS in the MFMA operand type;
//   2. the lower-triangular 16x16 tiles of K K^T and Q K^T on MFMA, masked
//      and scaled into A (fp32) and P = tril(Q K^T o G);
//   3. T = (I + A)^{-1}: 16x16 diagonal blocks by forward substitution in
//      fp32, off-diagonal blocks T_ij = -T_ii sum_m A_im T_mj on MFMA, one
//      block diagonal at a time;
//   4. per wave, with its state slab as the B operand: X = K S, Q S,
//      R = diag(beta)(V - gamma o X), E = T R, Y = gamma o QS + P E,
//      S = gamma_C S + Kt^T E. Accumulator tiles feed the next product's B
//      operand directly (see gdn_device.h), so E and R never touch LDS.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kChunkF32 = 64;

static __device__ __forceinline__ void tri_tile(int t, int &rt, int &ct) {
  // t = 0..9 -> lower-triangular tile (rt, ct) of a 4x4 tile grid, ct <= rt
  rt = (t >= 1) + (t >= 3) + (t >= 6);
  ct = t - rt * (rt + 1) / 2;
}

template <int DK, int DVT, typename TIN, typename TOUT, typename MT>
__global__ __launch_bounds__(64 * (DVT / 16)) void chunk_fwd_f32_kernel(
    const TIN *__restrict__ q, const TIN *__restrict__ k, const TIN *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    const float *__restrict__ gA, const float *__restrict__ gbias,
    const float *__restrict__ S0, TOUT *__restrict__ y, float *__restrict__ S_T,
    const int32_t *__restrict__ cu_seqlens, int T, int H, int DV, int n_vt, SegCtl seg) {
  constexpr int C = kChunkF32;
  constexpr int NW = DVT / 16;
  constexpr int NT = 64 * NW;
  constexpr int PAD = 16 / static_cast<int>(sizeof(MT));
  constexpr int LDK = DK + PAD;
  constexpr int LDC = C + PAD;
  constexpr int LDV = DVT + PAD;
  constexpr int LDA = C + 4;
  constexpr int NKT = DK / 16;
  constexpr int NKB = DK / 32;
  constexpr int VEC = io<TIN>::kVec;

  __shared__ __attribute__((aligned(16))) MT Ks[C * LDK];
  __shared__ __attribute__((aligned(16))) MT Qs[C * LDK];
  __shared__ __attribute__((aligned(16))) MT KtT[DK * LDC];
  __shared__ __attribute__((aligned(16))) MT Vs[C * LDV];
  __shared__ __attribute__((aligned(16))) MT Tm[C * LDC];
  __shared__ __attribute__((aligned(16))) MT Pm[C * LDC];
  __shared__ __attribute__((aligned(16))) float Am[C * LDA];
  __shared__ float s_g[C], s_gam[C], s_beta[C];

  int bid = blockIdx.x;
  const int vt = bid % n_vt;
  bid /= n_vt;
  const int h = bid % H;
  const int n = bid / H;

  int64_t bos, len;
  if (cu_seqlens) {
    int64_t a = cu_seqlens[n], b = cu_seqlens[n + 1];
    a = a < 0 ? 0 : (a > T ? T : a);
    b = b < a ? a : (b > T ? T : b);
    bos = a;
    len = b - a;
  } else {
    bos = static_cast<int64_t>(n) * T;
    len = T;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int v0 = vt * DVT;
  const int n0 = 16 * w;

  for (int i = tid; i < C * LDC; i += NT) {
    Tm[i] = (MT)0.0f;
    Pm[i] = (MT)0.0f;
  }

  // state slab: st[it][i] = S[16*it + 4*lg + i][v0 + n0 + lc]
  f32x4 st[NKT];
  const size_t sbase = static_cast<size_t>(n * H + h) * DK * DV + v0 + n0 + lc;
  const bool use_s0 = S0 != nullptr && n < seg.s0_nseq;
  const bool write_y = y != nullptr && n < seg.y_nseq;
#pragma unroll
  for (int it = 0; it < NKT; ++it)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * it + 4 * lg + i;
      st[it][i] = seg.s0_ident ? (row == v0 + n0 + lc ? 1.0f : 0.0f)
                  : use_s0     ? S0[sbase + static_cast<size_t>(row) * DV]
                               : 0.0f;
    }

  const RawGate gate = RawGate::load(gA, gbias, h);
  const int nchunks = static_cast<int>((len + C - 1) / C);
  for (int c = 0; c < nchunks; ++c) {
    const int64_t t0 = bos + static_cast<int64_t>(c) * C;
    const int valid = static_cast<int>(len - static_cast<int64_t>(c) * C < C
                                           ? len - static_cast<int64_t>(c) * C
                                           : C);

    // ---- 1. gates: every wave scans the chunk's 64 log-decays ----------
    float la = 0.0f, bt = 0.0f;
    if (lane < valid) {
      la = log_alpha[(t0 + lane) * H + h];
      bt = beta[(t0 + lane) * H + h];
      if (gate.raw()) {
        la = gate.log_alpha(la);
        bt = RawGate::beta(bt);
      }
    }
    float g = la;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(g, off, 64);
      if (lane >= off) g += o;
    }
    const float gC = __shfl(g, 63, 64);
    const float kdec = __expf(gC - g);  // exp(g_C - g_r) for r = lane

    __syncthreads();  // previous chunk is done with LDS
    if (w == 0) {
      s_g[lane] = g;
      s_gam[lane] = __expf(g);
      s_beta[lane] = bt;
    }

    // ---- K, Q (and Kt^T) and the V tile into LDS ------------------------
    constexpr int KV_PER_ROW = DK / VEC;
    constexpr int KV_TOTAL = C * KV_PER_ROW;
#pragma unroll
    for (int p = 0; p < (KV_TOTAL + NT - 1) / NT; ++p) {
      const int idx = tid + NT * p;
      const int r = (idx < KV_TOTAL ? idx : 0) / KV_PER_ROW;
      const int d0 = (idx % KV_PER_ROW) * VEC;
      const float kd = __shfl(kdec, r, 64);
      if (idx < KV_TOTAL) {
        float kv[VEC], qv[VEC];
        if (r < valid) {
          const size_t off = static_cast<size_t>((t0 + r) * H + h) * DK + d0;
          io<TIN>::load16(k + off, kv);
          io<TIN>::load16(q + off, qv);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) kv[e] = qv[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          Ks[r * LDK + d0 + e] = (MT)kv[e];
          Qs[r * LDK + d0 + e] = (MT)qv[e];
          KtT[(d0 + e) * LDC + r] = (MT)(kd * kv[e]);
        }
      }
    }
    constexpr int VV_PER_ROW = DVT / VEC;
    constexpr int VV_TOTAL = C * VV_PER_ROW;
#pragma unroll
    for (int p = 0; p < (VV_TOTAL + NT - 1) / NT; ++p) {
      const int idx = tid + NT * p;
      if (idx < VV_TOTAL) {
        const int r = idx / VV_PER_ROW;
        const int d0 = (idx % VV_PER_ROW) * VEC;
        float vv[VEC];
        if (r < valid && !seg.v_zero) {
          io<TIN>::load16(v + static_cast<size_t>((t0 + r) * H + h) * DV + v0 + d0, vv);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) vv[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) Vs[r * LDV + d0 + e] = (MT)vv[e];
      }
    }
    __syncthreads();

    // ---- 2. lower tiles of K K^T -> A (fp32), Q K^T -> P -----------------
    for (int tix = w; tix < 20; tix += NW) {
      const bool gram = tix < 10;
      int rt, ct;
      tri_tile(gram ? tix : tix - 10, rt, ct);
      const MT *X = gram ? Ks : Qs;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        Frag<MT> a, b;
        a.load_row(X, LDK, 16 * rt + lc, 32 * kb, lg);
        b.load_row(Ks, LDK, 16 * ct + lc, 32 * kb, lg);
        mma(acc, a, b);
      }
      const int col = 16 * ct + lc;
      const float gcol = s_g[col];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i;
        const float decay = __expf(fminf(s_g[r] - gcol, 0.0f));
        if (gram) {
          Am[r * LDA + col] = r > col ? s_beta[r] * decay * acc[i] : 0.0f;
        } else {
          Pm[r * LDC + col] = (MT)(r >= col ? decay * acc[i] : 0.0f);
        }
      }
    }
    __syncthreads();

    // ---- 3. T = (I + A)^{-1} ----------------------------------------------
    // diagonal blocks: lane (lg, lc) solves column lc of block lg
    if (w == 0) {
      const int b0 = 16 * lg;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == lc) ? 1.0f : 0.0f;
#pragma unroll
        for (int i = 0; i < r; ++i) acc = fmaf(-Am[(b0 + r) * LDA + b0 + i], x[i], acc);
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Tm[(b0 + r) * LDC + b0 + lc] = (MT)x[r];
    }
    __syncthreads();
    // off-diagonal blocks, one block diagonal (distance d) at a time
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      for (int j = w; j + d < 4; j += NW) {
        const int i = j + d;
        f32x4 M = zero4();
        for (int m = j; m < i; m += 2) {
          Frag<MT> a, b;
          if (m + 1 < i) {
            a.load_row_f32(Am, LDA, 16 * i + lc, 16 * m, lg);
            b.load_col(Tm, LDC, 16 * j + lc, 16 * m, lg);
          } else {
            Frag<MT> full;
            full.load_row_f32(Am, LDA, 16 * i + lc, 16 * m, lg);
            a = full;
#pragma unroll
            for (int s = 4; s < 8; ++s) a.v[s] = (MT)0.0f;
            b.load_col_lo(Tm, LDC, 16 * j + lc, 16 * m, lg);
          }
          mma(M, a, b);
        }
        Frag<MT> a, b;
        a.load_row_lo(Tm, LDC, 16 * i + lc, 16 * i, lg);
        b.from_acc_lo(M);
        f32x4 Tij = zero4();
        mma(Tij, a, b);
#pragma unroll
        for (int e = 0; e < 4; ++e) Tm[(16 * i + 4 * lg + e) * LDC + 16 * j + lc] = (MT)(-Tij[e]);
      }
      __syncthreads();
    }

    // ---- 4. state side, per wave on its 16-column slab --------------------
    Frag<MT> sb[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sb[kb].from_acc(st[2 * kb], st[2 * kb + 1]);

    f32x4 X[4], QS[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      X[rt] = zero4();
      QS[rt] = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        Frag<MT> a;
        a.load_row(Ks, LDK, 16 * rt + lc, 32 * kb, lg);
        mma(X[rt], a, sb[kb]);
        a.load_row(Qs, LDK, 16 * rt + lc, 32 * kb, lg);
        mma(QS[rt], a, sb[kb]);
      }
    }
    // R = beta (V - gamma X)
    f32x4 R[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i;
        R[rt][i] = s_beta[r] * (static_cast<float>(Vs[r * LDV + n0 + lc]) - s_gam[r] * X[rt][i]);
      }
    // E = T R
    Frag<MT> rb[2];
    rb[0].from_acc(R[0], R[1]);
    rb[1].from_acc(R[2], R[3]);
    f32x4 E[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      E[rt] = zero4();
#pragma unroll
      for (int kb = 0; kb <= rt / 2; ++kb) {
        Frag<MT> a;
        a.load_row(Tm, LDC, 16 * rt + lc, 32 * kb, lg);
        mma(E[rt], a, rb[kb]);
      }
    }
    Frag<MT> eb[2];
    eb[0].from_acc(E[0], E[1]);
    eb[1].from_acc(E[2], E[3]);
    // Y = gamma QS + P E
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 Y;
#pragma unroll
      for (int i = 0; i < 4; ++i) Y[i] = s_gam[16 * rt + 4 * lg + i] * QS[rt][i];
#pragma unroll
      for (int kb = 0; kb <= rt / 2; ++kb) {
        Frag<MT> a;
        a.load_row(Pm, LDC, 16 * rt + lc, 32 * kb, lg);
        mma(Y, a, eb[kb]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i;
        if (write_y && r < valid)
          y[static_cast<size_t>((t0 + r) * H + h) * DV + v0 + n0 + lc] = io<TOUT>::from_f32(Y[i]);
      }
    }
    // S = gamma_C S + Kt^T E
    const float gamC = s_gam[C - 1];
#pragma unroll
    for (int it = 0; it < NKT; ++it) {
      st[it] *= gamC;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<MT> a;
        a.load_row(KtT, LDC, 16 * it + lc, 32 * kb, lg);
        mma(st[it], a, eb[kb]);
      }
    }
  }

  if (S_T && n >= seg.st_first) {
    const size_t obase = static_cast<size_t>((n - seg.st_first) * H + h) * DK * DV + v0 + n0 + lc;
#pragma unroll
    for (int it = 0; it < NKT; ++it)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_T[obase + static_cast<size_t>(16 * it + 4 * lg + i) * DV] = st[it][i];
  }
}

template <int DK, int DVT, typename TIN, typename TOUT, typename MT>
static hipError_t launch_tile(const ChunkArgs &a) {
  const int n_vt = a.dv / DVT;
  const int64_t blocks = static_cast<int64_t>(a.N) * a.H * n_vt;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_fwd_f32_kernel<DK, DVT, TIN, TOUT, MT>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * (DVT / 16)), 0, a.stream, static_cast<const TIN *>(a.q),
                     static_cast<const TIN *>(a.k), static_cast<const TIN *>(a.v), a.log_alpha,
                     a.beta, a.A, a.b_alpha, a.S0, static_cast<TOUT *>(a.y), a.S_T, a.cu_seqlens, a.T, a.H, a.dv,
                     n_vt, a.seg);
  return hipGetLastError();
}

template <typename TOUT>
static hipError_t launch_f32_out(const ChunkArgs &a) {
  if (a.dk == 128) return launch_tile<128, 16, float, TOUT, float>(a);
  return launch_tile<64, 64, float, TOUT, float>(a);
}

hipError_t launch_chunk_fwd_f32(const ChunkArgs &a) {
  switch (a.out_dtype) {
    case 1: return launch_f32_out<bf16_t>(a);
    case 2: return launch_f32_out<_Float16>(a);
    default: return launch_f32_out<float>(a);
  }
}

}  // namespace gdn
