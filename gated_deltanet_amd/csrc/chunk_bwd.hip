// Chunked backward pass of the gated delta rule (gfx950).
//
// Gradients of L = <dy, y> + <dS_T, S_T> with respect to q, k, v, log alpha,
// beta and S0 for the recurrence of the page "NLP——技术报告解读-Qwen3.8-Flash-
// Next", section "Gated DeltaNet 核心机制" (the pages report backward kernels
// but print no formula; these are the derivatives of the chunk equations the
// forward evaluates). Per chunk of C tokens starting from state S, with g the
// in-chunk running sum of log alpha, gamma = e^g, G_ri = e^(g_r - g_i),
// A = strictly_lower(diag(beta)(K K^T o G)), T = (I + A)^-1, X = K S,
// R = diag(beta)(V - gamma o X), E = T R, P = tril(Q K^T o G),
// Kt_r = e^(g_C - g_r) k_r and dS' the gradient of the chunk-end state:
//     dE = Kt dS' + P^T dY,   dR = T^T dE,   dA = -strictly_lower(dR E^T),
//     dP = tril(dY E^T),      dV = diag(beta) dR,   dX = -diag(beta gamma) dR,
//     dQ = diag(gamma) dY S^T + (dP o G) K,
//     dK = diag(e^(g_C - g)) E dS'^T + (dP o G)^T Q + dX S^T + (N + N^T) K,
//          N = diag(beta)(dA o G),
//     dS = gamma_C dS' + (diag(gamma) Q)^T dY + K^T dX   (to the chunk before),
// and the gradient of g gathers every decay factor (gamma, G, Kt, gamma_C);
// d log alpha is its reverse running sum inside the chunk.
//
// The dS recurrence is separable by columns of the state, so one workgroup
// owns one (sequence, head, 32-column tile of S) and sweeps backward over the
// chunks, reading the tile's chunk-start states from a workspace. With
// 16-bit inputs the prefill kernel writes those states in a launch of its own
// just before; with fp32 inputs the workgroup first sweeps forward to rebuild
// them. dV and dS0 belong to the tile's columns
// and are written directly; dq, dk, dbeta and dlog alpha sum over all
// columns, so each tile writes its partial sums and a second kernel adds the
// tiles in a fixed order (no atomics: results are deterministic).
//
// Operands are staged in LDS in fp32. With fp32 inputs every product runs on
// v_mfma_f32_16x16x4_f32; with 16-bit inputs the operands are rounded to
// fp16 as fragments are loaded and run on v_mfma_f32_16x16x32_f16 (fp32
// accumulation). The work is split into phases separated by workgroup
// barriers, each phase's 16x16 output tiles dealt round-robin to the sixteen
// waves (four per SIMD).
#include <cstdlib>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kC = 32;     // chunk length
constexpr int kDVT = 32;   // state columns per workgroup
constexpr int kNT = 1024;  // threads
constexpr int kNW = 16;    // waves (four per SIMD, so one can issue while the others wait)
constexpr int kLDV = kDVT + 4;
constexpr int kLDC = kC + 4;

// 16x16 output tile (rows m0.., cols n0..) of a product with contraction
// length K (a multiple of 32). "row" operands are row-major with the
// contraction index contiguous; "col" operands are row-major with the
// contraction index as the row. Each fp32 fragment pair is 8 MFMAs; they
// go to four independent accumulators (summed at the end) so a wave does
// not wait on one long dependent chain.
struct Acc4 {
  f32x4 a[4];
  __device__ __forceinline__ Acc4() {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = zero4();
  }
  __device__ __forceinline__ void mma(const Frag<float> &x, const Frag<float> &y) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      a[j & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.v[j], y.v[j], a[j & 3], 0, 0, 0);
  }
  __device__ __forceinline__ void add_to(f32x4 &acc) const {
    acc += (a[0] + a[1]) + (a[2] + a[3]);
  }
};
// With 16-bit inputs (H16) the operands are rounded to fp16 as they are
// loaded and each fragment pair is one v_mfma_f32_16x16x32_f16 (fp32
// accumulation); fp32 inputs keep every product in fp32.
__device__ __forceinline__ void load_col_h(Frag<_Float16> &f, const float *base, int ld, int col,
                                           int r0, int lg) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.v[j] = (_Float16)base[(r0 + 4 * lg + j) * ld + col];
    f.v[4 + j] = (_Float16)base[(r0 + 16 + 4 * lg + j) * ld + col];
  }
}
template <bool H16>
__device__ __forceinline__ void mm_rr(f32x4 &acc, const float *A, int lda, const float *B, int ldb,
                                      int m0, int n0, int K, int lc, int lg) {
  if constexpr (H16) {
    for (int k0 = 0; k0 < K; k0 += 32) {
      Frag<_Float16> fa, fb;
      fa.load_row_f32(A, lda, m0 + lc, k0, lg);
      fb.load_row_f32(B, ldb, n0 + lc, k0, lg);
      mma(acc, fa, fb);
    }
  } else {
    Acc4 s;
    for (int k0 = 0; k0 < K; k0 += 32) {
      Frag<float> fa, fb;
      fa.load_row(A, lda, m0 + lc, k0, lg);
      fb.load_row(B, ldb, n0 + lc, k0, lg);
      s.mma(fa, fb);
    }
    s.add_to(acc);
  }
}
template <bool H16>
__device__ __forceinline__ void mm_rc(f32x4 &acc, const float *A, int lda, const float *B, int ldb,
                                      int m0, int n0, int K, int lc, int lg) {
  if constexpr (H16) {
    for (int k0 = 0; k0 < K; k0 += 32) {
      Frag<_Float16> fa, fb;
      fa.load_row_f32(A, lda, m0 + lc, k0, lg);
      load_col_h(fb, B, ldb, n0 + lc, k0, lg);
      mma(acc, fa, fb);
    }
  } else {
    Acc4 s;
    for (int k0 = 0; k0 < K; k0 += 32) {
      Frag<float> fa, fb;
      fa.load_row(A, lda, m0 + lc, k0, lg);
      fb.load_col(B, ldb, n0 + lc, k0, lg);
      s.mma(fa, fb);
    }
    s.add_to(acc);
  }
}
template <bool H16>
__device__ __forceinline__ void mm_cc(f32x4 &acc, const float *A, int lda, const float *B, int ldb,
                                      int m0, int n0, int K, int lc, int lg) {
  if constexpr (H16) {
    for (int k0 = 0; k0 < K; k0 += 32) {
      Frag<_Float16> fa, fb;
      load_col_h(fa, A, lda, m0 + lc, k0, lg);
      load_col_h(fb, B, ldb, n0 + lc, k0, lg);
      mma(acc, fa, fb);
    }
  } else {
    Acc4 s;
    for (int k0 = 0; k0 < K; k0 += 32) {
      Frag<float> fa, fb;
      fa.load_col(A, lda, m0 + lc, k0, lg);
      fb.load_col(B, ldb, n0 + lc, k0, lg);
      s.mma(fa, fb);
    }
    s.add_to(acc);
  }
}

// sum over the 16 lanes of a row of the wave (lanes with the same lane / 16)
__device__ __forceinline__ float sum16(float x) { return row_sum<16>(x); }

// 16 raw bytes of a 32- or 16-bit element type as floats
template <typename T>
__device__ __forceinline__ void raw16_to_f32(const u32x4 r, float *x) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(r[i]);
  } else if constexpr (std::is_same<T, bf16_t>::value) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(r[i] << 16);
      x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  } else {
    const f16x8 hv = __builtin_bit_cast(f16x8, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = static_cast<float>(hv[i]);
  }
}

// Sequence n's rows [bos, bos + len), the offsets clamped to [0, T].
__device__ __forceinline__ void seq_rows(const BwdArgs &a, int n, int64_t &bos, int64_t &len) {
  if (a.cu_seqlens) {
    int64_t s0 = a.cu_seqlens[n], s1 = a.cu_seqlens[n + 1];
    s0 = s0 < 0 ? 0 : (s0 > a.T ? a.T : s0);
    s1 = s1 < s0 ? s0 : (s1 > a.T ? a.T : s1);
    bos = s0;
    len = s1 - s0;
  } else {
    bos = static_cast<int64_t>(n) * a.T;
    len = a.T;
  }
}

// The chunks [c_lo, c_hi) of a sequence (first row bos, nc chunks) that run
// j sweeps (see BwdArgs::runs). Every chunk falls in exactly one run, and a
// later run never holds an earlier chunk.
__device__ __forceinline__ void run_chunks(const BwdArgs &a, int j, int64_t bos, int nc, int &c_lo,
                                           int &c_hi) {
  auto first = [&](int r) -> int {  // first chunk of run r
    if (r <= 0) return 0;
    if (r >= a.runs) return nc;
    if (a.run_rows == 0) return static_cast<int>(static_cast<int64_t>(r) * nc / a.runs);
    const int64_t row = static_cast<int64_t>(r) * a.run_rows;
    if (row <= bos) return 0;
    if (row >= bos + static_cast<int64_t>(nc) * kC) return nc;
    return static_cast<int>((row - bos + kC - 1) / kC);
  };
  c_lo = first(j);
  c_hi = first(j + 1);
}

// Rows a sequence (len rows, nc chunks) contributes to run j.
__device__ __forceinline__ int64_t run_seq_rows(const BwdArgs &a, int j, int64_t bos, int64_t len,
                                                int nc) {
  int c_lo, c_hi;
  run_chunks(a, j, bos, nc, c_lo, c_hi);
  if (c_lo >= c_hi) return 0;
  const int64_t end = static_cast<int64_t>(c_hi) * kC;
  return (end < len ? end : len) - static_cast<int64_t>(c_lo) * kC;
}

// Whether the runs' sequence offsets come from the run_off table: with
// more than one run, unless every sequence gives every run as many rows
// (equal lengths, proportional runs).
__device__ __host__ __forceinline__ bool run_table(const BwdArgs &a) {
  return a.runs > 1 && (a.cu_seqlens || a.run_rows > 0);
}

// Where sequence n's rows of run a.run start among the run's partial sums.
__device__ __forceinline__ int64_t run_seq_offset(const BwdArgs &a, int n, int64_t bos) {
  if (a.runs == 1) return bos;
  if (run_table(a)) return a.run_off[static_cast<size_t>(a.run) * (a.N + 1) + n];
  return static_cast<int64_t>(n) * run_seq_rows(a, a.run, 0, a.T, (a.T + kC - 1) / kC);
}

// Row j of the run offsets (see run_table): an exclusive scan
// of the sequences' row counts in run j = blockIdx.x, the total last.
__global__ __launch_bounds__(256) void run_offsets_kernel(const BwdArgs a) {
  const int j = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ int64_t sc[256];
  int64_t carry = 0;
  for (int base = 0; base < a.N; base += 256) {
    const int n = base + tid;
    int64_t cnt = 0;
    if (n < a.N) {
      int64_t bos, len;
      seq_rows(a, n, bos, len);
      cnt = run_seq_rows(a, j, bos, len, static_cast<int>((len + kC - 1) / kC));
    }
    sc[tid] = cnt;
    __syncthreads();
    for (int w = 1; w < 256; w <<= 1) {  // inclusive scan
      const int64_t x = tid >= w ? sc[tid - w] : 0;
      __syncthreads();
      sc[tid] += x;
      __syncthreads();
    }
    if (n < a.N)
      a.run_off[static_cast<size_t>(j) * (a.N + 1) + n] = static_cast<int32_t>(carry + sc[tid] - cnt);
    carry += sc[255];
    __syncthreads();
  }
  if (tid == 0) a.run_off[static_cast<size_t>(j) * (a.N + 1) + a.N] = static_cast<int32_t>(carry);
}

template <int DK, typename TIN, typename TG>
__global__ __launch_bounds__(kNT) void chunk_bwd_kernel(const BwdArgs a) {
  constexpr int C = kC, DVT = kDVT, LDV = kLDV, LDC = kLDC;
  constexpr int LDK = DK + 4;
  constexpr int NKT = DK / 16;  // 16-row tiles of the state
  constexpr int VEC = io<TIN>::kVec;
  constexpr bool H16 = sizeof(TIN) == 2;  // 16-bit inputs: fp16 operands
  using FragM = typename std::conditional<H16, Frag<_Float16>, Frag<float>>::type;

  __shared__ __attribute__((aligned(16))) float Ks[C * LDK];
  __shared__ __attribute__((aligned(16))) float Qs[C * LDK];
  __shared__ __attribute__((aligned(16))) float Vs[C * LDV];
  __shared__ __attribute__((aligned(16))) float dYs[C * LDV];
  __shared__ __attribute__((aligned(16))) float Ss[DK * LDV];
  __shared__ __attribute__((aligned(16))) float dSs[DK * LDV];
  __shared__ __attribute__((aligned(16))) float Xs[C * LDV];
  __shared__ __attribute__((aligned(16))) float Rs[C * LDV];
  __shared__ __attribute__((aligned(16))) float Es[C * LDV];
  __shared__ __attribute__((aligned(16))) float dEs[C * LDV];
  __shared__ __attribute__((aligned(16))) float dXs[C * LDV];
  // transposed copies (DVT rows of C) for the dS update's B operands
  // Both carry e^(g_r - g_0) = gamma_r / gamma_0 in place of gamma_r (at most
  // 1, the first row's exactly 1), and the product is scaled by gamma_0 in
  // fp32: with strong decay gamma_r itself can fall below the fp16 range of
  // the 16-bit operands, while the ratios keep the leading terms.
  __shared__ __attribute__((aligned(16))) float dYgt[DVT * LDC];  // (diag(gamma/gamma_0) dY)^T
  __shared__ __attribute__((aligned(16))) float dXt[DVT * LDC];   // (dX / gamma_0)^T
  // dR shares R's buffer: R is last read when E = T R is formed, one phase
  // before dR is written
  float *const dRs = Rs;
  __shared__ __attribute__((aligned(16))) float Am[C * LDC];   // A, strictly lower
  __shared__ __attribute__((aligned(16))) float Tm[C * LDC];   // (I + A)^-1
  __shared__ __attribute__((aligned(16))) float Pm[C * LDC];   // tril(Q K^T o G)
  __shared__ __attribute__((aligned(16))) float KGm[C * LDC];  // tril(K K^T o G)
  __shared__ __attribute__((aligned(16))) float dAm[C * LDC];
  __shared__ __attribute__((aligned(16))) float Mm[C * LDC];   // N + N^T, N = diag(beta)(dA o G)
  __shared__ __attribute__((aligned(16))) float dPm[C * LDC];
  __shared__ __attribute__((aligned(16))) float dPGm[C * LDC];  // dP o G
  __shared__ __attribute__((aligned(16))) float dPGt[C * LDC];  // (dP o G)^T
  __shared__ float s_g[C], s_gam[C], s_beta[C], s_kdec[C];
  __shared__ float s_qsdy[NKT][C], s_dbu[2][C], s_dgx[2][C], s_cr[NKT][C];
  __shared__ float s_db[C], s_red[kNW], s_colp[kNW][C];

  const TIN *__restrict__ q = static_cast<const TIN *>(a.q);
  const TIN *__restrict__ k = static_cast<const TIN *>(a.k);
  const TIN *__restrict__ v = static_cast<const TIN *>(a.v);
  const TG *__restrict__ dy = static_cast<const TG *>(a.dy);
  TG *__restrict__ dv_out = static_cast<TG *>(a.dv);
  const int H = a.H, DV = a.dv_size;
  const int n_vt = DV / DVT;

  // the n_vt column tiles of one (sequence, head) get ids that agree mod 8:
  // they run on one XCD and share its L2 for the K, Q and gate reads
  const int units = a.N * H;
  const int grp = blockIdx.x / (8 * n_vt);
  const int rem = blockIdx.x % (8 * n_vt);
  const int vt = rem / 8;
  const int unit = grp * 8 + rem % 8;
  if (unit >= units) return;
  const int h = unit % H;
  const int n = unit / H;
  int64_t bos, len;
  seq_rows(a, n, bos, len);
  const int nc = static_cast<int>((len + C - 1) / C);
  // this run's chunks, and the partial-sum row of sequence row t: t + pbase
  int c_lo, c_hi;
  run_chunks(a, a.run, bos, nc, c_lo, c_hi);
  const int64_t pbase =
      c_lo < c_hi ? run_seq_offset(a, n, bos) - bos - static_cast<int64_t>(c_lo) * C : 0;
  // chunk-state slots of this sequence: floor(bos / C) + n + c never
  // collide between sequences and stay below rows / C + N
  const int64_t slot0 = bos / C + n;

  // lane indices are re-made opaque at the start of every chunk (see
  // opaque_lanes): values derived from them are then recomputed inside the
  // chunk loops instead of being hoisted out of them and spilled
  int tid = threadIdx.x;
  int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int lc = lane & 15;
  int lg = lane >> 4;
  auto opaque_lanes = [&]() { asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lc), "+v"(lg)); };
  // one fragment of an fp32 LDS operand: row `row` (contraction along the
  // row) or column `col` (contraction down the column), from index k0
  auto ld_row = [&](FragM &f, const float *base, int ld, int row, int k0) {
    f.load_row_f32(base, ld, row, k0, lg);
  };
  auto ld_col = [&](FragM &f, const float *base, int ld, int col, int k0) {
    if constexpr (H16) load_col_h(f, base, ld, col, k0, lg);
    else f.load_col(base, ld, col, k0, lg);
  };
  const int v0 = vt * DVT;
  const size_t state_sz = static_cast<size_t>(DK) * DV;
  float *const ws_states = a.ws_states;
  const size_t part_stride = static_cast<size_t>(a.part_rows) * H;  // per tile, in rows*H
  // the state gradient of this tile between runs, [DK][DVT]
  float *const carry = a.ws_carry + (static_cast<size_t>(unit) * n_vt + vt) * (DK * DVT);
  if (c_lo == c_hi) {
    // no chunk in this run; a sequence without chunks gets dS0 = dS_T from
    // run 0
    if (nc == 0 && a.run == 0 && a.dS0)
      for (int idx = tid; idx < DK * DVT; idx += kNT) {
        const int r = idx / DVT, cc = idx % DVT;
        const size_t o = static_cast<size_t>(unit) * state_sz + r * DV + v0 + cc;
        a.dS0[o] = a.dS_T ? a.dS_T[o] : 0.0f;
      }
    return;
  }

  const RawGate gate = RawGate::load(a.A, a.b_alpha, h);
  // chunk-start state tiles in the workspace, [slot][head][column tile] blocks
  // of DK x DVT values in the accumulator order of state_row(): fp32 (rebuilt
  // here) with fp32 inputs, fp16 (from the prefill kernel) with 16-bit ones
  const size_t tile_idx0 = (static_cast<size_t>(slot0) * H + h) * n_vt + vt;
  auto state_tile = [&](int c) {  // fp32 inputs
    return ws_states + (tile_idx0 + static_cast<size_t>(c) * H * n_vt) * (DK * DVT);
  };
  auto state_tile16 = [&](int c) {  // 16-bit inputs
    return reinterpret_cast<const _Float16 *>(ws_states) +
           (tile_idx0 + static_cast<size_t>(c) * H * n_vt) * (DK * DVT);
  };
  // element e of the f32x4 with index idx of a state block: row and column
  auto state_rc = [&](int idx, int e, int &r, int &cc) {
    const int slab = idx / (DK / 16 * 64), t = (idx / 64) % (DK / 16), ln = idx % 64;
    r = state_row(t, ln >> 4, e);
    cc = 16 * slab + (ln & 15);
  };

  // ---- staging helpers ------------------------------------------------
  auto rows_valid = [&](int c) -> int {
    const int64_t r = len - static_cast<int64_t>(c) * C;
    return r >= C ? C : static_cast<int>(r);
  };
  // Chunk inputs are fetched into registers one chunk ahead (raw 16-byte
  // pieces, zeros past the sequence end) and staged into LDS at the start of
  // the chunk, so their HBM latency hides behind the previous chunk's work.
  constexpr int VG = io<TG>::kVec;
  constexpr int KI = (C * DK / VEC + kNT - 1) / kNT;      // K / Q pieces per thread
  constexpr int VI = (C * DVT / VEC + kNT - 1) / kNT;     // V pieces per thread
  constexpr int GI = (C * DVT / VG + kNT - 1) / kNT;      // dY pieces per thread
  constexpr int SI = (DK * DVT / 4 + kNT - 1) / kNT;      // state f32x4 per thread
  // Pieces are spread over the waves so that none issues (and stages) more
  // than three: K from thread 0, Q from thread kNT / 2 when it fits in half
  // the workgroup, V from thread 256, dY after it, the gates on the last wave.
  constexpr int KP = C * DK / VEC, VP = C * DVT / VEC, GP = C * DVT / VG;
  constexpr int QOFF = KP <= kNT / 2 ? kNT / 2 : 0;
  constexpr int VOFF = 256, GOFF = VOFF + (VP + 63) / 64 * 64;
  static_assert(VOFF + VP <= kNT && GOFF + GP <= kNT && VI == 1 && GI == 1,
                "V and dY pieces fit the workgroup once");
  constexpr int kGateWave = kNW - 1;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  struct Pre {
    u32x4 k[KI], q[KI], v[VI], dy[GI];
    f32x4 s[H16 ? 1 : SI];   // fp32 state pieces
    u32x2 sh[H16 ? SI : 1];  // fp16 state pieces (four values each)
    float la, bt;
  };
  const u32x4 zero_raw = {0u, 0u, 0u, 0u};
  // Every load goes through a buffer resource that covers the chunk's valid
  // rows (all heads), so rows past the sequence end and threads without a
  // piece (offset kNone) read zeros without a branch: with no branch around
  // the loads the compiler knows how many are in flight and waits for the
  // ones it needs, not for all of them.
  constexpr uint32_t kNone = 0x80000000u;
  auto rsrc = [](const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                             static_cast<int>(bytes), 0x00020000);
  };
  auto fetch = [&](Pre &p, int c, bool with_q, bool with_dy, bool with_state) {
    const int64_t t0 = bos + static_cast<int64_t>(c) * C;
    const int valid = rows_valid(c);
    const int64_t rows_b = static_cast<int64_t>(valid) * H;  // head-rows of the chunk
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      {
        const int idx = tid + kNT * i;
        const int r = idx / (DK / VEC), d0 = (idx % (DK / VEC)) * VEC;
        const uint32_t off = idx < KP ? static_cast<uint32_t>(((r * H + h) * DK + d0) * sizeof(TIN))
                                      : kNone;
        p.k[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rsrc(k + t0 * H * DK, rows_b * DK * sizeof(TIN)), off, 0, 0));
      }
      if (with_q) {
        const int idx = tid + kNT * i - QOFF;
        const int r = idx / (DK / VEC), d0 = (idx % (DK / VEC)) * VEC;
        const uint32_t off = (idx >= 0 && idx < KP)
                                 ? static_cast<uint32_t>(((r * H + h) * DK + d0) * sizeof(TIN))
                                 : kNone;
        p.q[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rsrc(q + t0 * H * DK, rows_b * DK * sizeof(TIN)), off, 0, 0));
      }
    }
    {
      const int idx = tid - VOFF;
      const int r = idx / (DVT / VEC), d0 = (idx % (DVT / VEC)) * VEC;
      const uint32_t off = (idx >= 0 && idx < VP)
                               ? static_cast<uint32_t>(((r * H + h) * DV + v0 + d0) * sizeof(TIN))
                               : kNone;
      p.v[0] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rsrc(v + t0 * H * DV, rows_b * DV * sizeof(TIN)), off, 0, 0));
    }
    if (with_dy) {
      const int idx = tid - GOFF;
      const int r = idx / (DVT / VG), d0 = (idx % (DVT / VG)) * VG;
      const uint32_t off = (idx >= 0 && idx < GP)
                               ? static_cast<uint32_t>(((r * H + h) * DV + v0 + d0) * sizeof(TG))
                               : kNone;
      p.dy[0] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rsrc(dy + t0 * H * DV, rows_b * DV * sizeof(TG)), off, 0, 0));
    }
    if (with_state) {
      // streamed once: non-temporal
      if constexpr (H16) {
        const auto rs = rsrc(state_tile16(c), DK * DVT * 2);
#pragma unroll
        for (int i = 0; i < SI; ++i) {
          const int idx = tid + kNT * i;
          const uint32_t off = idx < DK * DVT / 4 ? static_cast<uint32_t>(8 * idx) : kNone;
          p.sh[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 2));
        }
      } else {
        const auto rs = rsrc(state_tile(c), DK * DVT * 4);
#pragma unroll
        for (int i = 0; i < SI; ++i) {
          const int idx = tid + kNT * i;
          const uint32_t off = idx < DK * DVT / 4 ? static_cast<uint32_t>(16 * idx) : kNone;
          p.s[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
        }
      }
    }
    p.la = 0.0f;
    p.bt = 0.0f;
    if (wave == kGateWave) {
      const uint32_t off = lane < C ? static_cast<uint32_t>((lane * H + h) * 4) : kNone;
      p.la = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rsrc(a.log_alpha + t0 * H, rows_b * 4), off, 0, 0));
      p.bt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rsrc(a.beta + t0 * H, rows_b * 4), off, 0, 0));
    }
  };
  auto stage = [&](const Pre &p, int stage_valid, bool with_q, bool with_dy, bool with_state) {
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      float x[VEC];
      {
        const int idx = tid + kNT * i;
        if (idx < KP) {
          const int r = idx / (DK / VEC), d0 = (idx % (DK / VEC)) * VEC;
          raw16_to_f32<TIN>(p.k[i], x);
#pragma unroll
          for (int e = 0; e < VEC; ++e) Ks[r * LDK + d0 + e] = x[e];
        }
      }
      if (with_q) {
        const int idx = tid + kNT * i - QOFF;
        if (idx >= 0 && idx < KP) {
          const int r = idx / (DK / VEC), d0 = (idx % (DK / VEC)) * VEC;
          raw16_to_f32<TIN>(p.q[i], x);
#pragma unroll
          for (int e = 0; e < VEC; ++e) Qs[r * LDK + d0 + e] = x[e];
        }
      }
    }
    {
      const int idx = tid - VOFF;
      if (idx >= 0 && idx < VP) {
        const int r = idx / (DVT / VEC), d0 = (idx % (DVT / VEC)) * VEC;
        float x[VEC];
        raw16_to_f32<TIN>(p.v[0], x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) Vs[r * LDV + d0 + e] = x[e];
      }
    }
    if (with_dy) {
      const int idx = tid - GOFF;
      if (idx >= 0 && idx < GP) {
        const int r = idx / (DVT / VG), d0 = (idx % (DVT / VG)) * VG;
        float x[VG];
        raw16_to_f32<TG>(p.dy[0], x);
#pragma unroll
        for (int e = 0; e < VG; ++e) dYs[r * LDV + d0 + e] = x[e];
      }
    }
    if (with_state) {
#pragma unroll
      for (int i = 0; i < SI; ++i) {
        const int idx = tid + kNT * i;
        if (idx < DK * DVT / 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            int r, cc;
            state_rc(idx, e, r, cc);
            if constexpr (H16) {
              typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
              Ss[r * LDV + cc] = static_cast<float>(__builtin_bit_cast(f16x4, p.sh[i])[e]);
            } else {
              Ss[r * LDV + cc] = p.s[i][e];
            }
          }
        }
      }
    }
    // gates: the gate wave scans the chunk's log decays (rows past the end: 0)
    if (wave == kGateWave) {
      float g = p.la, bt = p.bt;
      if (gate.raw() && lane < stage_valid) {
        g = gate.log_alpha(g);
        bt = RawGate::beta(bt);
      }
      g = scan32(g, lane);
      const float gC = lane_value(g, C - 1);
      if (lane < C) {
        s_g[lane] = g;
        s_gam[lane] = __expf(g);
        s_beta[lane] = bt;
        s_kdec[lane] = __expf(gC - g);
      }
    }
  };
  auto decay = [&](int r, int i) { return __expf(fminf(s_g[r] - s_g[i], 0.0f)); };
  // the 3 lower 16x16 tiles of a 32x32 matrix: (0,0), (1,0), (1,1)
  auto low_tile = [](int t, int &rt, int &ct) {
    rt = t >= 1 ? 1 : 0;
    ct = t == 2 ? 1 : 0;
  };
  // T = (I + A)^-1 for C = 32 in two parts, each run by one wave. solve_diag:
  // the 16x16 diagonal blocks by forward substitution (each 16-lane row of the
  // wave solves one block, rows 2 and 3 repeat rows 0 and 1: lane lc holds
  // column lc of the block's A and T, and the substitution broadcasts A's
  // entries between lanes, unit_lower_solve16); the off-diagonal blocks are
  // set to zero. t10: T10 = -T11 (A10 T00) on the matrix cores, written over
  // the zero block.
  // block: 0 or 16 for one diagonal block (every DPP row of the wave solves
  // it), -1 for both (rows 0 and 2 solve the first, rows 1 and 3 the second)
  auto solve_diag = [&](int block) {
    const int b0 = block < 0 ? 16 * (lg & 1) : block;
    float ac[16], xv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ac[r] = Am[(b0 + r) * LDC + b0 + lc];
      xv[r] = (r == lc) ? 1.0f : 0.0f;
    }
    unit_lower_solve16(ac, xv);
    if (block < 0 ? lg < 2 : lg == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Tm[(b0 + r) * LDC + b0 + lc] = xv[r];
#pragma unroll
      for (int r = 0; r < 16; ++r) Tm[(b0 + r) * LDC + (16 - b0) + lc] = 0.0f;
    }
  };
  auto t10 = [&]() {
    // M = A10 T00 (16x16, contraction 16: the upper half of the slice is 0)
    f32x4 M = zero4();
    {
      Frag<float> fa, fb;
      fa.load_row_lo(Am, LDC, 16 + lc, 0, lg);
      fb.load_col_lo(Tm, LDC, lc, 0, lg);
      mma_lo(M, fa, fb);
    }
    f32x4 T10 = zero4();
    {
      Frag<float> fa, fb;
      fa.load_row_lo(Tm, LDC, 16 + lc, 16, lg);
      fb.from_acc_lo(M);
      mma_lo(T10, fa, fb);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) Tm[(16 + 4 * lg + i) * LDC + lc] = -T10[i];
  };
  // LDS written by this wave is read back by it: keep the compiler from
  // moving the reads ahead and wait for the writes (LDS serves a wave's
  // requests in order)
  auto lds_fence = [&]() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
  // issue priority of this wave on its SIMD (shared with three others): raised
  // for the serial chains that set a phase's length
  auto prio = [](bool high) {
    if (high) __builtin_amdgcn_s_setprio(2);
    else __builtin_amdgcn_s_setprio(0);
  };
  // column `col` of R = diag(beta)(V - diag(gamma) X) as a B fragment over
  // the chunk's 32 rows, formed from V and X as it is loaded
  auto ld_col_R = [&](FragM &f, int col) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = j < 4 ? 4 * lg + j : 16 + 4 * lg + (j - 4);
      const float rv = s_beta[r] * (Vs[r * LDV + col] - s_gam[r] * Xs[r * LDV + col]);
      if constexpr (H16) f.v[j] = (_Float16)rv;
      else f.v[j] = rv;
    }
  };

  // ======================= forward sweep: chunk-start states =============
  // With 16-bit inputs the prefill kernel has written them already (its
  // states output); fp32 inputs rebuild them here. Ss holds the tile of the
  // running state.
  Pre pf;
  if constexpr (!H16) {
  // (once per sequence: in the run that holds its last chunk, the first of
  // the runs that touch it)
  if (c_hi == nc) {
  for (int idx = tid; idx < DK * DVT; idx += kNT) {
    const int r = idx / DVT, cc = idx % DVT;
    Ss[r * LDV + cc] = a.S0 ? a.S0[static_cast<size_t>(unit) * state_sz + r * DV + v0 + cc] : 0.0f;
  }
  if (nc > 0) fetch(pf, 0, false, false, false);
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    opaque_lanes();
    {
      float *dst = state_tile(c);
      for (int idx = tid; idx < DK * DVT / 4; idx += kNT) {
        f32x4 sv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int r, cc;
          state_rc(idx, e, r, cc);
          sv[e] = Ss[r * LDV + cc];
        }
        *reinterpret_cast<f32x4 *>(dst + 4 * idx) = sv;
      }
    }
    stage(pf, rows_valid(c), false, false, false);
    __syncthreads();
    // A (3 tiles) and X = K S (4 tiles)
    for (int t = wave; t < 7; t += kNW) {
      f32x4 acc = zero4();
      if (t < 3) {
        int rt, ct;
        low_tile(t, rt, ct);
        mm_rr<H16>(acc, Ks, LDK, Ks, LDK, 16 * rt, 16 * ct, DK, lc, lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lg + i, col = 16 * ct + lc;
          Am[r * LDC + col] = r > col ? s_beta[r] * decay(r, col) * acc[i] : 0.0f;
        }
        if (rt == 1 && ct == 0) {  // the upper tile of A is zero
#pragma unroll
          for (int i = 0; i < 4; ++i) Am[(4 * lg + i) * LDC + 16 + lc] = 0.0f;
        }
      } else {
        const int rt = (t - 3) >> 1, nt = (t - 3) & 1;
        mm_rc<H16>(acc, Ks, LDK, Ss, LDV, 16 * rt, 16 * nt, DK, lc, lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) Xs[(16 * rt + 4 * lg + i) * LDV + 16 * nt + lc] = acc[i];
      }
    }
    __syncthreads();
    if (c + 1 < nc) fetch(pf, c + 1, false, false, false);
    if (wave == 0) {
      solve_diag(-1);
      lds_fence();
      t10();
    }
    // R = beta (V - gamma X), all threads
    for (int idx = tid; idx < C * DVT; idx += kNT) {
      const int r = idx / DVT, cc = idx % DVT;
      Rs[r * LDV + cc] = s_beta[r] * (Vs[r * LDV + cc] - s_gam[r] * Xs[r * LDV + cc]);
    }
    __syncthreads();
    // kdec o E, E = T R (4 tiles)
    for (int t = wave; t < 4; t += kNW) {
      const int rt = t >> 1, nt = t & 1;
      f32x4 acc = zero4();
      mm_rc<H16>(acc, Tm, LDC, Rs, LDV, 16 * rt, 16 * nt, C, lc, lg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i;
        Es[r * LDV + 16 * nt + lc] = s_kdec[r] * acc[i];
      }
    }
    __syncthreads();
    // S <- gamma_C S + K^T (kdec o E)  (NKT x 2 tiles, contraction over C)
    const float gamC = s_gam[C - 1];
    for (int t = wave; t < NKT * 2; t += kNW) {
      const int mt = t >> 1, nt = t & 1;
      f32x4 acc = zero4();
      mm_cc<H16>(acc, Ks, LDK, Es, LDV, 16 * mt, 16 * nt, C, lc, lg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float *p = Ss + (16 * mt + 4 * lg + i) * LDV + 16 * nt + lc;
        *p = gamC * *p + acc[i];
      }
    }
    __syncthreads();
  }
  }
  }

  // ======================= backward sweep ================================
  // from dS_T in the run that holds the sequence's last chunk, else from the
  // state gradient the previous run left
  for (int idx = tid; idx < DK * DVT; idx += kNT) {
    const int r = idx / DVT, cc = idx % DVT;
    dSs[r * LDV + cc] =
        c_hi < nc ? carry[idx]
                  : (a.dS_T ? a.dS_T[static_cast<size_t>(unit) * state_sz + r * DV + v0 + cc]
                            : 0.0f);
  }
  // dbeta and d log alpha of a finished chunk (first row t0c, nv valid rows,
  // gamma_C = gC) from the row and column sums its phases left in LDS; run
  // by the last wave while the next chunk's first phase keeps the others busy
  // (those sums are rewritten only from the fourth phase on).
  auto gate_grads = [&](int64_t t0c, int nv, float gC) {
    if (lane >= C) return;
    // d log alpha_s = sum_{r >= s} (gamma and X terms of d g_r)
    //               + sum_{r >= s} M_rs                  (decays G)
    //               + sum_{r < s} cr_r                   (Kt: e^(g_C - g_r))
    //               + gamma_C <S, dS'>                   (gamma_C)
    // The Kt terms enter d g_r with - and d g_C with +; the exclusive
    // prefix is what survives, again without forming the cancelling pair.
    const int r = lane;
    float rs = s_dgx[0][r] + s_dgx[1][r];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) rs += s_qsdy[kt][r];
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const float o = __shfl_down(rs, off, 64);
      if (r + off < C) rs += o;
    }
    float cr = 0.0f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) cr += s_cr[kt][r];
    float inc = cr;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const float o = __shfl_up(inc, off, 64);
      if (r >= off) inc += o;
    }
    const float ex = __shfl_up(inc, 1, 64);  // the previous lane's inclusive sum
    rs += r > 0 ? ex : 0.0f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) rs += s_colp[w][r];
    float sred = 0.0f;
#pragma unroll
    for (int w = 0; w < kNW / 2; ++w) sred += s_red[w];
    rs += gC * sred;
    if (r < nv) {
      float *dst = a.ws_part + static_cast<size_t>(2) * n_vt * part_stride * DK;
      dst[(static_cast<size_t>(vt) * 2) * part_stride + (t0c + r + pbase) * H + h] = s_db[r];
      dst[(static_cast<size_t>(vt) * 2 + 1) * part_stride + (t0c + r + pbase) * H + h] = rs;
    }
  };
  int64_t prev_t0 = 0;
  int prev_valid = 0;
  float prev_gamC = 0.0f;
  fetch(pf, c_hi - 1, true, true, true);
  for (int c = c_hi - 1; c >= c_lo; --c) {
    opaque_lanes();
    const int64_t t0 = bos + static_cast<int64_t>(c) * C;
    const int valid = rows_valid(c);
    stage(pf, valid, true, true, true);
    __syncthreads();

    // ---- P1 -------------------------------------------------------------
    // Eleven product tiles: P = tril(Q K^T o G) (0-2), X = K S (3-6) and
    // Kt dS' (7-10), on waves 0-8, 10 and 14. K K^T o G and A, one tile per
    // wave: 11 and 13 take a diagonal tile (rows 0-15, 16-31) and then solve
    // that diagonal block of T = (I + A)^-1, 12 the off-diagonal tile.
    // 15: gate gradients of the chunk before; 9 idle. Wave w runs on SIMD
    // w mod 4, so each solving wave shares its SIMD with two tile waves only.
    static_assert(kNW == 16, "the first phase deals its work to sixteen waves");
    auto gram_tile = [&](int t) {
      int rt, ct;
      low_tile(t, rt, ct);
      f32x4 acc = zero4();
      mm_rr<H16>(acc, Ks, LDK, Ks, LDK, 16 * rt, 16 * ct, DK, lc, lg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i, col = 16 * ct + lc;
        const float gv = r >= col ? decay(r, col) * acc[i] : 0.0f;
        KGm[r * LDC + col] = gv;
        Am[r * LDC + col] = r > col ? s_beta[r] * gv : 0.0f;
      }
      if (rt == 1 && ct == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int o = (4 * lg + i) * LDC + 16 + lc;
          KGm[o] = 0.0f;
          Am[o] = 0.0f;
        }
      }
    };
    if (wave == 15) {
      if (c < c_hi - 1) gate_grads(prev_t0, prev_valid, prev_gamC);
    } else if (wave == 11 || wave == 13) {
      prio(true);
      gram_tile(wave == 11 ? 0 : 2);
      lds_fence();
      solve_diag(wave == 11 ? 0 : 16);
      prio(false);
    } else if (wave == 12) {
      gram_tile(1);
    } else if (wave != 9) {
      const int t = wave < 9 ? wave : (wave == 10 ? 9 : 10);
      f32x4 acc = zero4();
      if (t < 3) {
        int rt, ct;
        low_tile(t, rt, ct);
        mm_rr<H16>(acc, Qs, LDK, Ks, LDK, 16 * rt, 16 * ct, DK, lc, lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lg + i, col = 16 * ct + lc;
          Pm[r * LDC + col] = r >= col ? decay(r, col) * acc[i] : 0.0f;
        }
        if (rt == 1 && ct == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) Pm[(4 * lg + i) * LDC + 16 + lc] = 0.0f;
        }
      } else {
        const bool isX = t < 7;  // X = K S, else Kt dS'
        const int rt = ((t - 3) % 4) >> 1, nt = (t - 3) & 1;
        mm_rc<H16>(acc, Ks, LDK, isX ? Ss : dSs, LDV, 16 * rt, 16 * nt, DK, lc, lg);
        if (isX) {
#pragma unroll
          for (int i = 0; i < 4; ++i) Xs[(16 * rt + 4 * lg + i) * LDV + 16 * nt + lc] = acc[i];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * lg + i;
            dEs[r * LDV + 16 * nt + lc] = s_kdec[r] * acc[i];
          }
        }
      }
    }
    __syncthreads();

    // ---- P2: E = T R (R formed on load); dE += P^T dY; gamma_C <S, dS'> ----
    // The two waves of E's lower row tile first complete T with T10 (both
    // write the same values). Tiles here and in the next phase are formed
    // transposed (operands swapped): lane (lg, lc) holds columns 4 lg ..
    // 4 lg + 3 of token row lc, one 16-byte LDS access.
    if (wave < 8) {
      const int t = wave;
      const int rt = (t & 3) >> 1, nt = t & 1;
      const int r = 16 * rt + lc, c4 = 16 * nt + 4 * lg;
      f32x4 acc = zero4();
      FragM fa, fb;
      if (t < 4) {
        if (rt == 1) {
          prio(true);
          t10();
          lds_fence();
        }
        ld_row(fa, Tm, LDC, r, 0);
        ld_col_R(fb, 16 * nt + lc);
        mma(acc, fb, fa);
        *reinterpret_cast<f32x4 *>(Es + r * LDV + c4) = acc;
        if (rt == 1) prio(false);
      } else {
        ld_col(fa, Pm, LDC, r, 0);
        ld_col(fb, dYs, LDV, 16 * nt + lc, 0);
        mma(acc, fb, fa);
        f32x4 *de = reinterpret_cast<f32x4 *>(dEs + r * LDV + c4);
        *de = *de + acc;
      }
    } else {
      // (diag(gamma / gamma_0) dY)^T for the dS update, and <S, dS'> over the
      // tile, one sum per wave, by the other eight waves
      for (int idx = tid - kNT / 2; idx < C * DVT; idx += kNT / 2) {
        const int r = idx / DVT, cc = idx % DVT;
        dYgt[cc * LDC + r] = __expf(s_g[r] - s_g[0]) * dYs[r * LDV + cc];
      }
      float acc = 0.0f;
      for (int idx = tid - kNT / 2; idx < DK * DVT; idx += kNT / 2) {
        const int r = idx / DVT, cc = idx % DVT;
        acc = fmaf(Ss[r * LDV + cc], dSs[r * LDV + cc], acc);
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) acc += __shfl_xor(acc, off, 64);
      if (lane == 0) s_red[wave - kNW / 2] = acc;
    }
    __syncthreads();

    // ---- P3: dR = T^T dE; dV, dX and their row sums; dP = tril(dY E^T) ---
    if (wave < 4) {
      const int t = wave;
      const int rt = t >> 1, nt = t & 1;
      const int r = 16 * rt + lc, c4 = 16 * nt + 4 * lg;  // transposed tile
      prio(true);
      f32x4 dr = zero4();
      {
        FragM fa, fb;
        ld_col(fa, Tm, LDC, r, 0);
        ld_col(fb, dEs, LDV, 16 * nt + lc, 0);
        mma(dr, fb, fa);
      }
      const float br = s_beta[r], gr = s_gam[r], bg = br * gr;
      const f32x4 x = *reinterpret_cast<const f32x4 *>(Xs + r * LDV + c4);
      const f32x4 vv = *reinterpret_cast<const f32x4 *>(Vs + r * LDV + c4);
      const f32x4 dx = -bg * dr;
      *reinterpret_cast<f32x4 *>(dRs + r * LDV + c4) = dr;
      *reinterpret_cast<f32x4 *>(dXs + r * LDV + c4) = dx;
      const float brel = -br * __expf(s_g[r] - s_g[0]);  // dX / gamma_0 per dR
#pragma unroll
      for (int e = 0; e < 4; ++e) dXt[(c4 + e) * LDC + r] = brel * dr[e];
      if (r < valid) {
        TG *dst = dv_out + ((t0 + r) * H + h) * DV + v0 + c4;
        if constexpr (sizeof(TG) == 4) {
          *reinterpret_cast<f32x4 *>(dst) = br * dr;
        } else {
          typedef TG tg4 __attribute__((ext_vector_type(4)));
          tg4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = io<TG>::from_f32(br * dr[e]);
          *reinterpret_cast<tg4 *>(dst) = o;
        }
      }
      // row sums over this tile's 16 columns: four in the lane, then the
      // four lane groups
      float su = 0.0f, sx = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        su += dr[e] * (vv[e] - gr * x[e]);
        sx += dx[e] * x[e];
      }
      su = xor32_sum(xor16_sum(su));
      sx = xor32_sum(xor16_sum(sx));
      if (lg == 0) {
        s_dbu[nt][r] = su;
        s_dgx[nt][r] = sx;
      }
      prio(false);
    } else if (wave < 7) {
      int rt, ct;
      low_tile(wave - 4, rt, ct);
      f32x4 acc = zero4();
      mm_rr<H16>(acc, dYs, LDV, Es, LDV, 16 * rt, 16 * ct, DVT, lc, lg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i, col = 16 * ct + lc;
        const float d = r >= col ? acc[i] : 0.0f;
        dPm[r * LDC + col] = d;
        const float dg = r >= col ? d * decay(r, col) : 0.0f;
        dPGm[r * LDC + col] = dg;
        dPGt[col * LDC + r] = dg;
      }
      if (rt == 1 && ct == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int o = (4 * lg + i) * LDC + 16 + lc;
          dPm[o] = 0.0f;
          dPGm[o] = 0.0f;
          dPGt[(16 + lc) * LDC + 4 * lg + i] = 0.0f;
        }
      }
    }
    __syncthreads();

    // ---- P4: dA = -strictly_lower(dR E^T); M = N + N^T ------------------
    if (wave < 3) {
      int rt, ct;
      low_tile(wave, rt, ct);
      f32x4 acc = zero4();
      mm_rr<H16>(acc, dRs, LDV, Es, LDV, 16 * rt, 16 * ct, DVT, lc, lg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i, col = 16 * ct + lc;
        // N is strictly lower: M = N + N^T gets N_rc at (r, c) and (c, r);
        // the entries above the diagonal come from the partner lane (or,
        // for the upper block, from the lower off-diagonal tile)
        const float d = r > col ? -acc[i] : 0.0f;
        dAm[r * LDC + col] = d;
        const float nv = s_beta[r] * d * decay(r, col);
        if (r > col) {
          Mm[r * LDC + col] = nv;
          Mm[col * LDC + r] = nv;
        } else if (r == col) {
          Mm[r * LDC + col] = 0.0f;
        }
      }
      if (rt == 1 && ct == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dAm[(4 * lg + i) * LDC + 16 + lc] = 0.0f;
      }
    }
    __syncthreads();

    // the next chunk's inputs, fetched before this phase's partial stores:
    // a later wait for a store (before its data registers are reused) would
    // also wait for loads issued after it
    if (c > c_lo) fetch(pf, c - 1, true, true, true);

    // ---- P5: partial dQ and dK, one (row tile, key tile) pair per wave --
    // The pair's dQ and dK tiles share the S row fragment (dY S^T, dX S^T)
    // and the K column fragment ((dP o G) K, (N + N^T) K). Both tiles are
    // formed transposed (operands swapped): lane (lg, lc) then holds keys
    // 4 lg .. 4 lg + 3 of token row lc, stored with one 16-byte write.
    for (int t = wave; t < 2 * NKT; t += kNW) {
      const int rt = t / NKT, kt = t % NKT;
      const int r = 16 * rt + lc;      // token row of this lane
      const int k4 = 16 * kt + 4 * lg; // its first key
      FragM fS, fK, fa, fb;
      ld_row(fS, Ss, LDV, 16 * kt + lc, 0);
      ld_col(fK, Ks, LDK, 16 * kt + lc, 0);
      // dQ = diag(gamma) dY S^T + (dP o G) K. The gamma terms of d g,
      // gamma_r (Q S)_r . dY_r = gamma_r sum_k Q_rk (dY S^T)_rk, are sums of
      // Q o (dY S^T) over the row's keys: four in the lane, then the four
      // lane groups.
      f32x4 acc = zero4();
      ld_row(fa, dYs, LDV, r, 0);
      mma(acc, fS, fa);
      acc *= s_gam[r];
      {
        const f32x4 qv = *reinterpret_cast<const f32x4 *>(Qs + r * LDK + k4);
        float qs = (acc[0] * qv[0] + acc[1] * qv[1]) + (acc[2] * qv[2] + acc[3] * qv[3]);
        qs = xor32_sum(xor16_sum(qs));
        if (lg == 0) s_qsdy[kt][r] = qs;
      }
      ld_row(fa, dPGm, LDC, r, 0);
      mma(acc, fK, fa);
      // dK = diag(kdec) E dS'^T + (dP o G)^T Q + dX S^T + (N + N^T) K
      f32x4 acc2 = zero4();
      ld_row(fa, Es, LDV, r, 0);
      ld_row(fb, dSs, LDV, 16 * kt + lc, 0);
      mma(acc2, fb, fa);
      acc2 *= s_kdec[r];
      {
        const f32x4 kv = *reinterpret_cast<const f32x4 *>(Ks + r * LDK + k4);
        float cr = (acc2[0] * kv[0] + acc2[1] * kv[1]) + (acc2[2] * kv[2] + acc2[3] * kv[3]);
        cr = xor32_sum(xor16_sum(cr));
        if (lg == 0) s_cr[kt][r] = cr;
      }
      ld_row(fa, dPGt, LDC, r, 0);
      ld_col(fb, Qs, LDK, 16 * kt + lc, 0);
      mma(acc2, fb, fa);
      ld_row(fa, dXs, LDV, r, 0);
      mma(acc2, fS, fa);
      ld_row(fa, Mm, LDC, r, 0);
      mma(acc2, fK, fa);
      if (r < valid) {
        const size_t o = ((t0 + r + pbase) * H + h) * DK + k4;
        *reinterpret_cast<f32x4 *>(a.ws_part + static_cast<size_t>(vt) * part_stride * DK + o) = acc;
        *reinterpret_cast<f32x4 *>(a.ws_part + (static_cast<size_t>(n_vt) + vt) * part_stride * DK +
                                   o) = acc2;
      }
    }
    // Row work for dbeta and d log alpha, one (row r, column i) element of
    // the 32x32 chunk matrices per thread (a wave holds two rows).
    // The decay factors G_ri = e^(g_r - g_i) contribute W_ri = dP_ri P_ri +
    // dA_ri A_ri to d g_r and -W_ri to d g_i; summed into d log alpha_s =
    // sum_{r >= s} d g_r, every W_ri with both indices >= s cancels, leaving
    // sum_{r >= s} sum_{i < s} W_ri. That sum is formed directly (row prefix
    // M_rs = sum_{i < s} W_ri, then column sums over r >= s) instead of adding
    // and subtracting terms that cancel, which loses everything in fp32 when
    // the true gradient is tiny (strong decay).
    {
      static_assert(kNT == C * C, "one thread per element of a chunk matrix");
      const int r = tid >> 5, i = tid & 31;
      const int o = r * LDC + i;
      // dbeta_r: the beta (V - gamma X) terms plus sum_i dA_ri (K K^T o G)_ri
      float db = row_sum<16>(dAm[o] * KGm[o]);
      db = xor16_sum(db);
      if (i == 0) s_db[r] = db + s_dbu[0][r] + s_dbu[1][r];
      const float w = i < r ? dPm[o] * Pm[o] + dAm[o] * Am[o] : 0.0f;
      // inclusive prefix along the row (32 lanes), then shifted by one lane:
      // M_ri = the previous lane's inclusive sum (0 at i = 0); the first lane
      // of a DPP row takes the last of the row before
      const float inc = scan32(w, lane);
      const float last15 = lane_value(inc, 15), last47 = lane_value(inc, 47);
      float m = row_shr<1>(inc);
      if (i == 16) m = lane < 32 ? last15 : last47;
      // column i gets M_ri from every row r >= i; the wave's two rows first
      float col = r >= i ? m : 0.0f;
      col = xor32_sum(col);
      if (lane < 32) s_colp[wave][i] = col;
    }
    __syncthreads();


    // ---- P6: dS <- gamma_C dS' + (diag(gamma) Q)^T dY + K^T dX -----------
    const float gamC = s_gam[C - 1], gam0 = s_gam[0];
    for (int t = wave; t < NKT * 2; t += kNW) {
      const int mt = t >> 1, nt = t & 1;
      // A operands: columns of Q and K (contraction over the chunk's rows);
      // B operands: rows of the transposed copies, relative to gamma_0
      f32x4 acc = zero4();
      FragM fa, fb;
      ld_col(fa, Qs, LDK, 16 * mt + lc, 0);
      ld_row(fb, dYgt, LDC, 16 * nt + lc, 0);
      mma(acc, fa, fb);
      ld_col(fa, Ks, LDK, 16 * mt + lc, 0);
      ld_row(fb, dXt, LDC, 16 * nt + lc, 0);
      mma(acc, fa, fb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float *p = dSs + (16 * mt + 4 * lg + i) * LDV + 16 * nt + lc;
        *p = gamC * *p + gam0 * acc[i];
      }
    }
    prev_t0 = t0;
    prev_valid = valid;
    prev_gamC = gamC;
    __syncthreads();
  }
  if (wave == kNW - 1) gate_grads(prev_t0, prev_valid, prev_gamC);
  // dS0 for this tile after the sequence's first chunk, else the carry to
  // the next run
  if (c_lo == 0) {
    if (a.dS0)
      for (int idx = tid; idx < DK * DVT; idx += kNT) {
        const int r = idx / DVT, cc = idx % DVT;
        a.dS0[static_cast<size_t>(unit) * state_sz + r * DV + v0 + cc] = dSs[r * LDV + cc];
      }
  } else {
    for (int idx = tid; idx < DK * DVT; idx += kNT) {
      const int r = idx / DVT, cc = idx % DVT;
      carry[idx] = dSs[r * LDV + cc];
    }
  }
}

// The sequence row of partial-sum row p of run a.run, or -1 for a row that
// holds nothing.
__device__ __forceinline__ int64_t run_row(const BwdArgs &a, int64_t p) {
  if (a.runs == 1) return p < a.rows ? p : -1;
  int n;
  int64_t off;
  if (run_table(a)) {
    // the last sequence whose rows start at or before p
    const int32_t *o = a.run_off + static_cast<size_t>(a.run) * (a.N + 1);
    if (p >= o[a.N]) return -1;
    int lo = 0, hi = a.N;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (o[mid] <= p) lo = mid;
      else hi = mid;
    }
    n = lo;
    off = o[lo];
  } else {
    const int64_t per = run_seq_rows(a, a.run, 0, a.T, (a.T + kC - 1) / kC);
    if (per == 0 || p >= per * a.N) return -1;
    n = static_cast<int>(p / per);
    off = per * n;
  }
  int64_t bos, len;
  seq_rows(a, n, bos, len);
  int c_lo, c_hi;
  run_chunks(a, a.run, bos, static_cast<int>((len + kC - 1) / kC), c_lo, c_hi);
  return bos + static_cast<int64_t>(c_lo) * kC + (p - off);
}

// Sum of the column tiles' partial dq, dk (C x dk rows) and dbeta, dlog
// alpha, in tile order, for the rows of one run.
template <int DK, int NVT, typename TG>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const BwdArgs a) {
  constexpr int n_vt = NVT;  // column tiles (dv / 32)
  const size_t part_stride = static_cast<size_t>(a.part_rows) * a.H;
  const size_t total_k = part_stride * DK;
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  // dq, dk: four consecutive elements per thread (16-byte partial loads)
  const int64_t rk = 4 * i < total_k ? run_row(a, static_cast<int64_t>(4 * i / (a.H * DK))) : -1;
  if (rk >= 0) {
    // every partial is read once: all loads issued before the sums, streamed
    f32x4 pq[NVT], pk[NVT];
#pragma unroll
    for (int t = 0; t < NVT; ++t) {
      pq[t] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4 *>(a.ws_part + static_cast<size_t>(t) * total_k + 4 * i));
      pk[t] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(
          a.ws_part + static_cast<size_t>(NVT + t) * total_k + 4 * i));
    }
    f32x4 sq = zero4(), sk = zero4();
#pragma unroll
    for (int t = 0; t < NVT; ++t) {  // tiles in order: deterministic
      sq += pq[t];
      sk += pk[t];
    }
    const size_t o = static_cast<size_t>(rk) * a.H * DK + 4 * i % (static_cast<size_t>(a.H) * DK);
    TG *dq = static_cast<TG *>(a.dq) + o;
    TG *dk = static_cast<TG *>(a.dk) + o;
    if constexpr (sizeof(TG) == 4) {
      *reinterpret_cast<f32x4 *>(dq) = sq;
      *reinterpret_cast<f32x4 *>(dk) = sk;
    } else {
      typedef TG tg4 __attribute__((ext_vector_type(4)));
      tg4 q4, k4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        q4[e] = io<TG>::from_f32(sq[e]);
        k4[e] = io<TG>::from_f32(sk[e]);
      }
      *reinterpret_cast<tg4 *>(dq) = q4;
      *reinterpret_cast<tg4 *>(dk) = k4;
    }
  }
  if (i < part_stride) {
    float *g = a.ws_part + static_cast<size_t>(2) * n_vt * total_k;
    const int64_t rg = run_row(a, static_cast<int64_t>(i / a.H));
    if (rg < 0) {
      // rows that hold nothing add nothing to the per-head sums
      if (a.A) g[i] = g[part_stride + i] = 0.0f;
      return;
    }
    const size_t gi = static_cast<size_t>(rg) * a.H + i % a.H;
    float sb = 0.0f, sl = 0.0f;
    for (int t = 0; t < n_vt; ++t) {
      sb += g[(static_cast<size_t>(t) * 2) * part_stride + i];
      sl += g[(static_cast<size_t>(t) * 2 + 1) * part_stride + i];
    }
    if (a.A) {
      // chain rule through log alpha = -e^A softplus(a + b_alpha) and
      // beta = sigmoid(b); the per-row terms of dA and db_alpha go over
      // tile 0's partials (this thread has read them) for the head sums
      const int h = static_cast<int>(gi % a.H);
      const RawGate gate = RawGate::load(a.A, a.b_alpha, h);
      const float x = a.log_alpha[gi] + gate.bias;
      const float sig = 1.0f / (1.0f + expf(-x));
      const float da = sl * (-gate.scale * sig);
      const float bt = RawGate::beta(a.beta[gi]);
      a.dbeta[gi] = sb * bt * (1.0f - bt);
      a.dlog_alpha[gi] = da;
      g[i] = sl * gate.log_alpha(a.log_alpha[gi]);
      g[part_stride + i] = da;
    } else {
      a.dbeta[gi] = sb;
      a.dlog_alpha[gi] = sl;
    }
  }
}

// Per-head sums over rows of the raw-gate terms (dA and db_alpha): one
// workgroup per head, each thread sums rows in order, then a fixed tree.
__global__ __launch_bounds__(256) void head_sum_kernel(const BwdArgs a) {
  const int h = blockIdx.x;
  const int n_vt = a.dv_size / kDVT;
  const size_t part_stride = static_cast<size_t>(a.part_rows) * a.H;
  const float *g = a.ws_part + static_cast<size_t>(2) * n_vt * part_stride * a.dk_size;
  float s0 = 0.0f, s1 = 0.0f;
  for (int64_t r = threadIdx.x; r < a.part_rows; r += 256) {
    s0 += g[r * a.H + h];
    s1 += g[part_stride + r * a.H + h];
  }
  __shared__ float red[2][256];
  red[0][threadIdx.x] = s0;
  red[1][threadIdx.x] = s1;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      red[0][threadIdx.x] += red[0][threadIdx.x + w];
      red[1][threadIdx.x] += red[1][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {  // the runs' sums are added in run order
    const bool first = a.run == a.runs - 1;
    a.dA[h] = (first ? 0.0f : a.dA[h]) + red[0][0];
    a.db_alpha[h] = (first ? 0.0f : a.db_alpha[h]) + red[1][0];
  }
}

}  // namespace

// Runs of the backward: the column tiles' partial sums are kept for one run
// at a time, at most about kBwdPartBytes of them (some 3 000 rows at H = 16,
// d = 128); a problem whose partials fit is one run. Each run costs about
// one chunk step more (the sweep's pipeline refills), so the bound trades
// workspace against time. Runs that take the same
// share of every sequence keep every sequence busy in every run; they are
// used while a chunk of every sequence is a small part of a run, and runs of
// consecutive rows (which hold many short sequences each) otherwise.
constexpr size_t kBwdPartBytes = size_t{192} << 20;

BwdSegPlan bwd_seg_plan(int64_t rows, int N, int H, int dk, int dv) {
  const size_t per_row = static_cast<size_t>(dv / kDVT) * H * (2 * dk + 2) * sizeof(float);
  BwdSegPlan p{1, 0, rows < 0 ? 0 : rows};
  if (rows <= 0 || N <= 0 || per_row == 0) return p;
  // GDN_BWD_RUNS (proportional runs) or GDN_BWD_SEGMENT_ROWS (runs of that
  // many rows, rounded down to whole chunks) set the runs instead, so that
  // tests reach both forms on small problems
  int64_t runs = 0, seg = 0;
  if (const char *e = getenv("GDN_BWD_RUNS")) runs = atoll(e);
  if (const char *e = getenv("GDN_BWD_SEGMENT_ROWS")) seg = atoll(e) / kC * kC;
  const int64_t cap = static_cast<int64_t>(kBwdPartBytes / per_row);
  const int64_t padded = rows + static_cast<int64_t>(N) * (kC - 1);  // rows in whole chunks, at most
  if (runs <= 0 && seg <= 0) {
    if (rows <= cap) return p;
    if (2 * static_cast<int64_t>(N) * kC <= cap)
      runs = (padded + cap - static_cast<int64_t>(N) * kC - 1) / (cap - static_cast<int64_t>(N) * kC);
    else
      seg = cap - kC;
  }
  if (runs > 0) {
    if (runs == 1) return p;
    // a sequence gives a run at most ceil(nc / runs) chunks
    p.runs = static_cast<int>(runs);
    const int64_t bound = (padded + runs - 1) / runs + static_cast<int64_t>(N) * kC;
    p.part_rows = bound < rows ? bound : rows;
    return p;
  }
  seg = seg < kC ? kC : seg / kC * kC;
  if (seg >= rows) return p;
  p.run_rows = seg;
  p.runs = static_cast<int>((rows + seg - 1) / seg);
  // a chunk that starts in a run's rows may end up to C - 1 rows past them
  p.part_rows = seg + kC < rows ? seg + kC : rows;
  return p;
}

namespace {

template <int DK, typename TIN, typename TG>
hipError_t launch_bwd_t(const BwdArgs &a) {
  const int n_vt = a.dv_size / kDVT;
  const int64_t units = static_cast<int64_t>(a.N) * a.H;
  if (units > 0) {
    if constexpr (sizeof(TIN) == 2) {
      // chunk-start states from the prefill kernel (no y, no final state)
      ChunkArgs f{};
      f.q = a.q;
      f.k = a.k;
      f.v = a.v;
      f.log_alpha = a.log_alpha;
      f.beta = a.beta;
      f.A = a.A;
      f.b_alpha = a.b_alpha;
      f.S0 = a.S0;
      f.y = nullptr;
      f.S_T = nullptr;
      f.cu_seqlens = a.cu_seqlens;
      f.N = a.N;
      f.T = a.T;
      f.H = a.H;
      f.dk = DK;
      f.dv = a.dv_size;
      f.in_dtype = a.in_dtype;
      f.out_dtype = a.in_dtype;
      f.stream = a.stream;
      f.states = a.ws_states;
      const hipError_t e = launch_chunk_fwd_states(f);
      if (e != hipSuccess) return e;
    }
  }
  // the sweep, the tile reduction and the per-head sums once per run, the
  // last chunks first (the state gradient flows backwards)
  const BwdSegPlan sp = bwd_seg_plan(a.rows, a.N, a.H, DK, a.dv_size);
  BwdArgs r = a;
  r.runs = sp.runs;
  r.run_rows = sp.run_rows;
  r.part_rows = sp.part_rows;
  if (run_table(r) && a.N > 0) {
    hipLaunchKernelGGL(run_offsets_kernel, dim3(sp.runs), dim3(256), 0, a.stream, r);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (int j = sp.runs - 1; j >= 0; --j) {
    BwdArgs b = r;
    b.run = j;
    if (units > 0) {
      const int64_t blocks = (units + 7) / 8 * 8 * n_vt;
      hipLaunchKernelGGL((chunk_bwd_kernel<DK, TIN, TG>), dim3(static_cast<unsigned>(blocks)),
                         dim3(kNT), 0, b.stream, b);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const size_t total = static_cast<size_t>(b.part_rows) * b.H * DK;
    if (total > 0) {
      // one thread per four dq/dk elements, which also covers the rows * H
      // gate rows (DK >= 4)
      const dim3 grid(static_cast<unsigned>((total / 4 + 255) / 256));
      if (b.dv_size == 128)
        hipLaunchKernelGGL((bwd_reduce_kernel<DK, 128 / kDVT, TG>), grid, dim3(256), 0, b.stream, b);
      else
        hipLaunchKernelGGL((bwd_reduce_kernel<DK, 64 / kDVT, TG>), grid, dim3(256), 0, b.stream, b);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (b.A) hipLaunchKernelGGL(head_sum_kernel, dim3(b.H), dim3(256), 0, b.stream, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TIN, typename TG>
hipError_t launch_bwd_d(const BwdArgs &a) {
  return a.dk_size == 128 ? launch_bwd_t<128, TIN, TG>(a) : launch_bwd_t<64, TIN, TG>(a);
}

template <typename TIN>
hipError_t launch_bwd_g(const BwdArgs &a) {
  switch (a.grad_dtype) {
    case 1: return launch_bwd_d<TIN, bf16_t>(a);
    case 2: return launch_bwd_d<TIN, _Float16>(a);
    default: return launch_bwd_d<TIN, float>(a);
  }
}

}  // namespace

// Workspace: the chunk-start states (one slot per chunk, floor(bos / C) + n
// + c for chunk c of sequence n), then the column tiles' partial sums of one
// run, then (with more than one run) the state gradients carried between
// runs and the runs' sequence offsets.
size_t chunk_bwd_states_bytes(int64_t rows, int N, int H, int dk, int dv, int in_dtype) {
  const size_t slots = static_cast<size_t>(rows / kC + N);
  // fp32 states for fp32 inputs, fp16 for 16-bit inputs
  const size_t states = slots * H * dk * dv * (in_dtype == 0 ? sizeof(float) : sizeof(_Float16));
  return (states + 255) / 256 * 256;
}

BwdLayout chunk_bwd_layout(int64_t rows, int N, int H, int dk, int dv, int in_dtype) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const BwdSegPlan p = bwd_seg_plan(rows, N, H, dk, dv);
  BwdLayout l;
  l.part = chunk_bwd_states_bytes(rows, N, H, dk, dv, in_dtype);
  const size_t n_vt = static_cast<size_t>(dv / kDVT);
  l.carry = l.part + up(n_vt * static_cast<size_t>(p.part_rows) * H * (2 * dk + 2) * sizeof(float));
  l.table = l.carry + (p.runs > 1 ? up(static_cast<size_t>(N) * H * dk * dv * sizeof(float)) : 0);
  l.total = l.table + (p.runs > 1 ? up(static_cast<size_t>(p.runs) * (N + 1) * sizeof(int32_t)) : 0);
  return l;
}

size_t chunk_bwd_workspace_size(int64_t rows, int N, int H, int dk, int dv, int in_dtype) {
  if (rows < 0 || N < 0 || H <= 0) return 0;
  return chunk_bwd_layout(rows, N, H, dk, dv, in_dtype).total;
}

hipError_t launch_chunk_bwd(const BwdArgs &a) {
  switch (a.in_dtype) {
    case 1: return launch_bwd_g<bf16_t>(a);
    case 2: return launch_bwd_g<_Float16>(a);
    default: return launch_bwd_g<float>(a);
  }
}

}  // namespace gdn
