// Chunked parallel prefill of the gated delta rule, bf16 inputs (gfx950).
//
// Math (page "NLP——技术报告解读-Qwen3.8-Flash-Next", section "Gated DeltaNet
// 核心机制", unrolled over a chunk). Inside a chunk of C tokens that starts
// from state S, with g_r the in-chunk running sum of log alpha,
// gamma_r = exp(g_r), G_ri = exp(g_r - g_i) (r >= i) and E the matrix of
// beta-scaled prediction errors:
//     A = strictly_lower(diag(beta) (K K^T o G)),   T = (I + A)^{-1}
//     X = K S,   R = diag(beta) (V - diag(gamma) X),   E = T R
//     Y = diag(gamma) (Q S) + tril(Q K^T o G) E
//     S <- gamma_C S + Kt^T E,   Kt_r = exp(g_C - g_r) k_r
// T is the UT transform of the compact WY form of the chunk's product of
// (I - beta k k^T) factors. Only exponentials of non-positive numbers occur.
//
// Work split. One workgroup owns one (sequence, head, 16*NS-column slice of
// the state) and walks the sequence's chunks in order. It has NS "state"
// waves and two "prep" waves:
//   * the state waves keep their 16-column slab of the fp32 state in
//     registers for the whole sequence and run the serial part: X = K S
//     (bf16 MFMA, A operands straight from the raw K tile), Q S (fp16 MFMA on
//     queries converted to fp16 in place by a prep wave), R, E = T R,
//     Y = gamma QS + P E and the state update (fp16 MFMA);
//   * the prep waves run one chunk ahead and produce, for the next chunk,
//     everything that does not depend on the state: the gate scan, T (Gram
//     tiles on MFMA, 16x16 diagonal blocks by forward substitution in fp32,
//     off-diagonal blocks on MFMA), P = tril(Q K^T o G), and Kt^T (the
//     transpose is done on the matrix cores with a 0/1 selector operand, so
//     it is exact).
//   * raw K, Q, V and gate tiles are streamed from HBM into a ring of LDS
//     slots by direct-to-LDS loads (global_load_lds_dwordx4) issued R-1
//     chunks ahead, so HBM latency overlaps with compute. One workgroup
//     barrier per chunk hands a finished chunk from the prep waves to the
//     state waves.
//
// Operand layouts in LDS are "fragment-linear": a 16x32 MFMA operand slice is
// stored as 64 lanes x 16 bytes, lane L's eight values contiguous at 16*L, so
// every operand read is one conflict-free ds_read_b128. To make the raw K/Q
// rows land that way straight from HBM, the key dimension inside each
// 32-slice is visited in the order 8*lg + j for lane group lg and slot j, and
// the state rows are stored in the matching order (see state_row()).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kC = 32;     // tokens per chunk
constexpr int kNCT = 2;    // 16-token tiles per chunk
constexpr int kRing = 6;   // raw-tile ring slots
constexpr int kDepth = kRing - 1;  // chunks of prefetch issued ahead

// LDS layout (bytes) for key size DK and NS state waves.
template <int DK, int NS>
struct Lay {
  static constexpr int DVT = 16 * NS;
  static constexpr int NKB = DK / 32;  // 32-deep key slices
  static constexpr int NST = DK / 16;  // 16-row state tiles
  // ring slot: raw bf16 tiles of one chunk
  static constexpr int K_OFF = 0;
  static constexpr int Q_OFF = K_OFF + kNCT * NKB * 1024;
  static constexpr int V_OFF = Q_OFF + kNCT * NKB * 1024;
  static constexpr int G_OFF = V_OFF + kC * DVT * 2;  // log_alpha[32], beta[32]
  static constexpr int SLOT = G_OFF + 256;
  // processed buffer (double-buffered): prep -> state hand-off
  static constexpr int T_OFF = 0;                      // T, kNCT fragments
  static constexpr int P_OFF = T_OFF + kNCT * 1024;    // P, kNCT fragments
  static constexpr int KT_OFF = P_OFF + kNCT * 1024;   // Kt^T, NST fragments
  static constexpr int GM_OFF = KT_OFF + NST * 1024;   // gamma[32]
  static constexpr int BT_OFF = GM_OFF + kC * 4;       // beta[32]
  static constexpr int PROC = BT_OFF + kC * 4;
  // prep-private fp32 scratch for the UT inverse
  static constexpr int LDA = kC + 4;  // A^T, row stride (floats)
  static constexpr int LDT = kC + 1;  // T, row stride (floats)
  static constexpr int RING = 0;
  static constexpr int PROCB = RING + kRing * SLOT;
  static constexpr int AMT = PROCB + 2 * PROC;
  static constexpr int TMP = AMT + kC * LDA * 4;
  static constexpr int FAC = TMP + kC * LDT * 4;  // decay factors, 2 x 128 floats
  static constexpr int TOTAL = FAC + 2 * 128 * 4;
  // direct-to-LDS loads per chunk issued by each prep wave
  static constexpr int NV = kC * DVT * 2 / 1024;  // V tile, 1 KiB per load
  static constexpr int LOADS_P0 = kNCT * NKB + 1; // K + gates
  static constexpr int LOADS_P1 = kNCT * NKB + NV; // Q + V
  static_assert(kC * DVT * 2 % 1024 == 0, "V tile must be whole KiB");
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// state tile t, lane group lg, element i  ->  key index
__device__ __forceinline__ int state_row(int t, int lg, int i) {
  return 32 * (t >> 1) + 8 * lg + 4 * (t & 1) + i;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  // generic -> LDS address-space conversion yields the 32-bit LDS offset
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char *)(p)));
}

// Direct-to-LDS loads: lane L's data lands at (M0 + 16*L) or (M0 + 4*L).
// Written in asm so the compiler does not serialise later LDS reads behind
// them; completion is tracked explicitly with vmcnt waits.
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// workgroup barrier that does not drain outstanding direct-to-LDS loads
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ float dpp_shr(float x) {
  // row_shr:N within 16-lane rows; lanes without a source read 0
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, true));
}
__device__ __forceinline__ float readlane(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

__device__ __forceinline__ f32x4 mma_bf16(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f16(const f16x8 &a, const f16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 pack_f16(const f32x4 &a, const f32x4 &b) {
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = (_Float16)a[j];
    r[4 + j] = (_Float16)b[j];
  }
  return r;
}
__device__ __forceinline__ bf16x8 pack_bf16(const f32x4 &a, const f32x4 &b) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = (__bf16)a[j];
    r[4 + j] = (__bf16)b[j];
  }
  return r;
}
__device__ __forceinline__ void store_out(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16_t *p, float v) {
  *reinterpret_cast<__bf16 *>(p) = (__bf16)v;  // v_cvt_pk_bf16_f32, round to nearest even
}
__device__ __forceinline__ void store_out(_Float16 *p, float v) { *p = (_Float16)v; }

// Operations on the raw 16-bit input tiles (K, Q, V) for each input type.
// bf16 inputs keep bf16 operands for the key-side products (exact inputs;
// the state operand of K S is rounded to bf16) and have Q converted to fp16
// by a prep wave for Q S; fp16 inputs use fp16 operands throughout.
template <typename TIN>
struct KOps;
template <>
struct KOps<bf16_t> {
  typedef bf16x8 vec;
  static constexpr bool kConvertQ = true;
  __device__ static f32x4 mma(const vec &a, const vec &b, f32x4 c) { return mma_bf16(a, b, c); }
  __device__ static vec pack(const f32x4 &a, const f32x4 &b) { return pack_bf16(a, b); }
  __device__ static float to_f32(uint16_t bits) { return bf16_to_f32(bits); }
};
template <>
struct KOps<_Float16> {
  typedef f16x8 vec;
  static constexpr bool kConvertQ = false;
  __device__ static f32x4 mma(const vec &a, const vec &b, f32x4 c) { return mma_f16(a, b, c); }
  __device__ static vec pack(const f32x4 &a, const f32x4 &b) { return pack_f16(a, b); }
  __device__ static float to_f32(uint16_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, bits));
  }
};

template <typename V>
__device__ __forceinline__ V lds_read16(const char *p) {
  return *reinterpret_cast<const V *>(p);
}

template <int DK, int NS, typename TIN, typename TOUT>
__global__ __launch_bounds__(64 * (NS + 2)) void chunk_fwd_bf16_kernel(
    const TIN *__restrict__ q, const TIN *__restrict__ k, const TIN *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    const float *__restrict__ S0, TOUT *__restrict__ y, float *__restrict__ S_T,
    const int32_t *__restrict__ cu_seqlens, int T, int H, int DV, int n_vt, int n_units) {
  using L = Lay<DK, NS>;
  using KO = KOps<TIN>;
  using kvec = typename KO::vec;
  constexpr int NKB = L::NKB;
  constexpr int NST = L::NST;
  constexpr int DVT = L::DVT;
  __shared__ __attribute__((aligned(1024))) char smem[L::TOTAL];

  // Workgroups are dealt to the 8 XCDs round-robin by id. The n_vt column
  // tiles of one (sequence, head) read the same K, Q and gates, so they are
  // given ids that agree mod 8: they run on one XCD and share its L2.
  const int units = n_units;
  const int grp = blockIdx.x / (8 * n_vt);
  const int rem = blockIdx.x % (8 * n_vt);
  const int vt = rem / 8;
  const int unit = grp * 8 + rem % 8;
  if (unit >= units) return;
  const int h = unit % H;
  const int n = unit / H;
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
  const int nc = static_cast<int>((len + kC - 1) / kC);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int v0 = vt * DVT;
  const bool is_state = wave < NS;
  const bool is_p0 = wave == NS;  // gates, Gram, UT inverse
  const int slab = 16 * wave;     // state waves: first column of the slab

  char *const ring = smem + L::RING;
  char *const procb = smem + L::PROCB;
  float *const amt = reinterpret_cast<float *>(smem + L::AMT);
  float *const tmp = reinterpret_cast<float *>(smem + L::TMP);

  // zero the parts of the hand-off buffers that are never rewritten (upper
  // blocks of P) and the prep scratch for T (its upper block stays zero)
  for (int i = threadIdx.x; i < 2 * L::PROC / 4; i += 64 * (NS + 2))
    reinterpret_cast<float *>(procb)[i] = 0.0f;
  for (int i = threadIdx.x; i < kC * L::LDT; i += 64 * (NS + 2)) tmp[i] = 0.0f;

  // ---- prep: issue the direct-to-LDS loads of chunk x into its ring slot --
  // Rows past the end of the sequence are clamped to its last row (in
  // bounds; their contributions are masked by beta = 0 and the store mask),
  // so every call issues the same number of loads and the vmcnt arithmetic
  // below holds even for chunk indices past the end.
  auto issue_chunk = [&](int x) {
    char *slot = ring + (x % kRing) * L::SLOT;
    const int64_t last = bos + len - 1;
    if (is_p0) {
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt) {
        int64_t row = bos + static_cast<int64_t>(x) * kC + 16 * rt + lc;
        row = row > last ? last : row;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          dma16(k + (row * H + h) * DK + 32 * kb + 8 * lg,
                lds_addr(slot + L::K_OFF + (rt * NKB + kb) * 1024));
      }
      int64_t row = bos + static_cast<int64_t>(x) * kC + (lane & 31);
      row = row > last ? last : row;
      dma4((lane < 32 ? log_alpha : beta) + row * H + h, lds_addr(slot + L::G_OFF));
    } else {
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt) {
        int64_t row = bos + static_cast<int64_t>(x) * kC + 16 * rt + lc;
        row = row > last ? last : row;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          dma16(q + (row * H + h) * DK + 32 * kb + 8 * lg,
                lds_addr(slot + L::Q_OFF + (rt * NKB + kb) * 1024));
      }
#pragma unroll
      for (int p = 0; p < L::NV; ++p) {
        const int qi = 64 * p + lane;
        const int r = qi / (DVT / 8);
        const int cc = qi % (DVT / 8);
        int64_t row = bos + static_cast<int64_t>(x) * kC + r;
        row = row > last ? last : row;
        dma16(v + (row * H + h) * DV + v0 + 8 * cc, lds_addr(slot + L::V_OFF + p * 1024));
      }
    }
  };

  // ---- prep: gate scan and decay factors -----------------------------------
  // Running sums are kept in log2 units (g2 = g / ln 2) so every decay is a
  // single v_exp_f32. Within a chunk the decay G_rc = 2^(g2_r - g2_c) factors
  // as a_r * b_c with a_r = 2^(g2_r - g2_m), b_c = 2^(g2_m - g2_c) around the
  // middle token m; that replaces one exponential per matrix element by one
  // per row. The factorisation is used only when both factors stay well
  // inside the fp32 range; otherwise (extreme gates) the chunk falls back to
  // one exponential per element. The branch is uniform per chunk.
  struct Gates {
    float g2, bt, gC2, gm2;
    bool fast;
  };
  auto scan_gates = [&](const char *slot, int x, float *fac, Gates &G) {
    const float *gl = reinterpret_cast<const float *>(slot + L::G_OFF);
    const int64_t tok = static_cast<int64_t>(x) * kC + lane;
    float la = 0.0f, bt = 0.0f;
    if (lane < kC && tok < len) {
      la = gl[lane];
      bt = gl[32 + lane];
    }
    float sc = la * 1.4426950408889634f;
    sc += dpp_shr<1>(sc);
    sc += dpp_shr<2>(sc);
    sc += dpp_shr<4>(sc);
    sc += dpp_shr<8>(sc);
    const float r15 = readlane(sc, 15);
    if (lane >= 16) sc += r15;
    G.g2 = sc;
    G.bt = bt;
    G.gC2 = readlane(sc, kC - 1);
    G.gm2 = r15;
    const float g0 = readlane(sc, 0);
    G.fast = (g0 - G.gm2 <= 120.0f) && (G.gm2 - G.gC2 <= 120.0f);
    if (lane < kC) {
      fac[64 + lane] = sc;
      fac[96 + lane] = bt;
      fac[32 + lane] = __builtin_amdgcn_exp2f(G.gm2 - sc);  // b_c
    }
  };
  // ---- prep wave 0: gates, Gram -> A, T = (I + A)^{-1} ---------------------
  float *const fac0 = reinterpret_cast<float *>(smem + L::FAC);
  float *const fac1 = fac0 + 128;
  auto prep0 = [&](int x) {
    const char *slot = ring + (x % kRing) * L::SLOT;
    char *pb = procb + (x & 1) * L::PROC;
    Gates G;
    scan_gates(slot, x, fac0, G);
    if (lane < kC) {
      reinterpret_cast<float *>(pb + L::GM_OFF)[lane] = __builtin_amdgcn_exp2f(G.g2);
      reinterpret_cast<float *>(pb + L::BT_OFF)[lane] = G.bt;
      fac0[lane] = G.bt * __builtin_amdgcn_exp2f(G.g2 - G.gm2);  // beta_r a_r
    }
    kvec kf[kNCT][NKB];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        kf[rt][kb] = lds_read16<kvec>(slot + L::K_OFF + (rt * NKB + kb) * 1024 + 16 * lane);
    f32x4 gram[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) gram[t] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      gram[0] = KO::mma(kf[0][kb], kf[0][kb], gram[0]);
      gram[1] = KO::mma(kf[1][kb], kf[0][kb], gram[1]);
      gram[2] = KO::mma(kf[1][kb], kf[1][kb], gram[2]);
    }
    wait_lds();
    f32x4 rf[kNCT];
    float cf[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) {
      rf[rt] = *reinterpret_cast<const f32x4 *>(fac0 + 16 * rt + 4 * lg);
      cf[rt] = fac0[32 + 16 * rt + lc];
    }
    // A = strictly_lower(diag(beta) (K K^T o G)), stored transposed in fp32
    f32x4 av[3];
    if (G.fast) {
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int rt = t == 0 ? 0 : 1, ct = t == 2 ? 1 : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) av[t][i] = rf[rt][i] * cf[ct] * gram[t][i];
      }
    } else {
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int rt = t == 0 ? 0 : 1, ct = t == 2 ? 1 : 0;
        const f32x4 gr = *reinterpret_cast<const f32x4 *>(fac0 + 64 + 16 * rt + 4 * lg);
        const f32x4 br = *reinterpret_cast<const f32x4 *>(fac0 + 96 + 16 * rt + 4 * lg);
        const float gc = fac0[64 + 16 * ct + lc];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[t][i] = br[i] * __builtin_amdgcn_exp2f(fminf(gr[i] - gc, 0.0f)) * gram[t][i];
      }
    }
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int rt = t == 0 ? 0 : 1, ct = t == 2 ? 1 : 0;
      const int c = 16 * ct + lc;
      f32x4 a;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = (16 * rt + 4 * lg + i > c) ? av[t][i] : 0.0f;
      *reinterpret_cast<f32x4 *>(amt + c * L::LDA + 16 * rt + 4 * lg) = a;
    }
    wait_lds();
    // diagonal 16x16 blocks of T by forward substitution, one column per lane
    {
      const int b = lg & (kNCT - 1);
      float xv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) xv[r] = (r == lc) ? 1.0f : 0.0f;
#pragma unroll
      for (int sidx = 0; sidx < 15; ++sidx) {
        const float *arow = amt + (16 * b + sidx) * L::LDA + 16 * b;  // A[16b + r][16b + s]
        float av[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4 t4 = *reinterpret_cast<const f32x4 *>(arow + 4 * u);
          av[4 * u] = t4[0];
          av[4 * u + 1] = t4[1];
          av[4 * u + 2] = t4[2];
          av[4 * u + 3] = t4[3];
        }
        const float xs = xv[sidx];
#pragma unroll
        for (int r = sidx + 1; r < 16; ++r) xv[r] = fmaf(-av[r], xs, xv[r]);
      }
      if (lg < kNCT) {
#pragma unroll
        for (int r = 0; r < 16; ++r) tmp[(16 * b + r) * L::LDT + 16 * b + lc] = xv[r];
      }
    }
    wait_lds();
    // off-diagonal block: T_10 = -T_11 (A_10 T_00)
    {
      f16x8 a, bb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = (_Float16)amt[(4 * lg + j) * L::LDA + 16 + lc];  // A[16 + lc][4 lg + j]
        bb[j] = (_Float16)tmp[(4 * lg + j) * L::LDT + lc];        // T_00[4 lg + j][lc]
        a[4 + j] = (_Float16)0.0f;
        bb[4 + j] = (_Float16)0.0f;
      }
      const f32x4 M = mma_f16(a, bb, zero4());
      f16x8 t11, mb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        t11[j] = (_Float16)tmp[(16 + lc) * L::LDT + 16 + 4 * lg + j];
        mb[j] = (_Float16)M[j];
        t11[4 + j] = (_Float16)0.0f;
        mb[4 + j] = (_Float16)0.0f;
      }
      const f32x4 D = mma_f16(t11, mb, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) tmp[(16 + 4 * lg + i) * L::LDT + lc] = -D[i];
    }
    wait_lds();
    // T in fragment-linear fp16: row 16 mt + lc, slot j <-> token 16(j>>2) + 4 lg + (j&3)
#pragma unroll
    for (int mt = 0; mt < kNCT; ++mt) {
      f16x8 f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        f[j] = (_Float16)tmp[(16 * mt + lc) * L::LDT + 16 * (j >> 2) + 4 * lg + (j & 3)];
      *reinterpret_cast<f16x8 *>(pb + L::T_OFF + mt * 1024 + 16 * lane) = f;
    }
  };

  // ---- prep wave 1: P = tril(Q K^T o G), Q -> fp16, Kt^T ------------------
  // 0/1 selector operand for exact transposes on the matrix cores: in lane
  // (lg, lc), slot j is 1 iff lg == lc >> 2 and j == 4u + (lc & 3).
  kvec sel[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sel[u][j] = (lg == (lc >> 2) && j == 4 * u + (lc & 3)) ? 1.0f : 0.0f;

  auto prep1 = [&](int x) {
    char *slot = ring + (x % kRing) * L::SLOT;
    char *pb = procb + (x & 1) * L::PROC;
    Gates G;
    scan_gates(slot, x, fac1, G);
    const float kdec = __builtin_amdgcn_exp2f(G.gC2 - G.g2);
    if (lane < kC) fac1[lane] = __builtin_amdgcn_exp2f(G.g2 - G.gm2);  // a_r
    kvec kf[kNCT][NKB], qf[kNCT][NKB];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        kf[rt][kb] = lds_read16<kvec>(slot + L::K_OFF + (rt * NKB + kb) * 1024 + 16 * lane);
        qf[rt][kb] = lds_read16<kvec>(slot + L::Q_OFF + (rt * NKB + kb) * 1024 + 16 * lane);
      }
    f32x4 qk[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) qk[t] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      qk[0] = KO::mma(qf[0][kb], kf[0][kb], qk[0]);
      qk[1] = KO::mma(qf[1][kb], kf[0][kb], qk[1]);
      qk[2] = KO::mma(qf[1][kb], kf[1][kb], qk[2]);
    }
    // Q in fp16 for the state waves' Q S: D_u = Sel_u x Q^T puts keys
    // 8 lg + 4u + i of token lc in lane (lg, lc), i.e. the A-operand slots;
    // exact, then rounded from bf16 values that fp16 represents exactly.
    // Written back over the raw Q of this slot, which no other wave reads
    // during this chunk step.
    if constexpr (KO::kConvertQ) {
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const f32x4 d0 = KO::mma(sel[0], qf[rt][kb], zero4());
        const f32x4 d1 = KO::mma(sel[1], qf[rt][kb], zero4());
        *reinterpret_cast<f16x8 *>(slot + L::Q_OFF + (rt * NKB + kb) * 1024 + 16 * lane) =
            pack_f16(d0, d1);
      }
    }
    wait_lds();
    f32x4 rf[kNCT];
    float cf[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) {
      rf[rt] = *reinterpret_cast<const f32x4 *>(fac1 + 16 * rt + 4 * lg);
      cf[rt] = fac1[32 + 16 * rt + lc];
    }
    // P: lower tiles, written straight into fragment-linear positions
    f32x4 pv[3];
    if (G.fast) {
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int rt = t == 0 ? 0 : 1, ct = t == 2 ? 1 : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[t][i] = rf[rt][i] * cf[ct] * qk[t][i];
      }
    } else {
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int rt = t == 0 ? 0 : 1, ct = t == 2 ? 1 : 0;
        const f32x4 gr = *reinterpret_cast<const f32x4 *>(fac1 + 64 + 16 * rt + 4 * lg);
        const float gc = fac1[64 + 16 * ct + lc];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pv[t][i] = __builtin_amdgcn_exp2f(fminf(gr[i] - gc, 0.0f)) * qk[t][i];
      }
    }
    _Float16 *pm = reinterpret_cast<_Float16 *>(pb + L::P_OFF);
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int rt = t == 0 ? 0 : 1, ct = t == 2 ? 1 : 0;
      const int c = 16 * ct + lc;
      const int jc = 4 * (ct & 1) + (lc & 3);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i;
        const int ldst = 16 * (lc >> 2) + 4 * lg + i;  // destination lane
        pm[(rt * 64 + ldst) * 8 + jc] = (_Float16)(r >= c ? pv[t][i] : 0.0f);
      }
    }
    // Kt^T: for each state tile, transpose 16 keys x 32 tokens on the matrix
    // cores and scale token columns by exp(g_C - g_t)
    float kd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kd[j] = __shfl(kdec, 16 * (j >> 2) + 4 * lg + (j & 3), 64);
#pragma unroll
    for (int t = 0; t < NST; ++t) {
      const f32x4 d0 = KO::mma(kf[0][t >> 1], sel[t & 1], zero4());
      const f32x4 d1 = KO::mma(kf[1][t >> 1], sel[t & 1], zero4());
      f16x8 f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[j] = (_Float16)(kd[j] * d0[j]);
        f[4 + j] = (_Float16)(kd[4 + j] * d1[j]);
      }
      *reinterpret_cast<f16x8 *>(pb + L::KT_OFF + t * 1024 + 16 * lane) = f;
    }
  };

  // ---- state waves: registers ---------------------------------------------
  f32x4 st[NST];
  const size_t sbase = static_cast<size_t>(n * H + h) * DK * DV + v0 + slab + lc;
  if (is_state) {
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st[t][i] = S0 ? S0[sbase + static_cast<size_t>(state_row(t, lg, i)) * DV] : 0.0f;
  }

  auto state_step = [&](int x) {
    const char *slot = ring + (x % kRing) * L::SLOT;
    const char *pb = procb + (x & 1) * L::PROC;
    // every LDS operand of this chunk, issued up front (one wave per SIMD:
    // nothing else would hide their latency)
    kvec kf[kNCT][NKB];
    f16x8 qf[kNCT][NKB], tf[kNCT], pf[kNCT], ktf[NST];
    f32x4 G4[kNCT], B4[kNCT];
    uint16_t vraw[kNCT][4];
    const float *gam = reinterpret_cast<const float *>(pb + L::GM_OFF);
    const float *bet = reinterpret_cast<const float *>(pb + L::BT_OFF);
    const uint16_t *vt_ = reinterpret_cast<const uint16_t *>(slot + L::V_OFF);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt)
        kf[rt][kb] = lds_read16<kvec>(slot + L::K_OFF + (rt * NKB + kb) * 1024 + 16 * lane);
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) {
      G4[rt] = *reinterpret_cast<const f32x4 *>(gam + 16 * rt + 4 * lg);
      B4[rt] = *reinterpret_cast<const f32x4 *>(bet + 16 * rt + 4 * lg);
#pragma unroll
      for (int i = 0; i < 4; ++i) vraw[rt][i] = vt_[(16 * rt + 4 * lg + i) * DVT + slab + lc];
      tf[rt] = lds_read16<f16x8>(pb + L::T_OFF + rt * 1024 + 16 * lane);
    }
    const float gC = gam[kC - 1];
#pragma unroll
    for (int t = 0; t < NST; ++t) ktf[t] = lds_read16<f16x8>(pb + L::KT_OFF + t * 1024 + 16 * lane);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt)
        qf[rt][kb] = lds_read16<f16x8>(slot + L::Q_OFF + (rt * NKB + kb) * 1024 + 16 * lane);
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) pf[rt] = lds_read16<f16x8>(pb + L::P_OFF + rt * 1024 + 16 * lane);

    // the state as B operand: bf16 against the raw bf16 keys for X = K S,
    // fp16 against the fp16 queries for Q S (Q S feeds y directly, so it gets
    // the finer rounding; errors in X are largely corrected by the delta rule)
    kvec sb[NKB];
    f16x8 sh[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sb[kb] = KO::pack(st[2 * kb], st[2 * kb + 1]);
      sh[kb] = pack_f16(st[2 * kb], st[2 * kb + 1]);
    }
    // serial chain: X = K S -> R -> E = T R -> S update
    f32x4 X[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) X[rt] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt) X[rt] = KO::mma(kf[rt][kb], sb[kb], X[rt]);
    f32x4 QS[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) QS[rt] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt) QS[rt] = mma_f16(qf[rt][kb], sh[kb], QS[rt]);
    f32x4 R[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        R[rt][i] = B4[rt][i] * (KO::to_f32(vraw[rt][i]) - G4[rt][i] * X[rt][i]);
    const f16x8 rb = pack_f16(R[0], R[1]);
    f32x4 E[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) E[rt] = mma_f16(tf[rt], rb, zero4());
    const f16x8 eb = pack_f16(E[0], E[1]);
#pragma unroll
    for (int t = 0; t < NST; ++t) st[t] = mma_f16(ktf[t], eb, st[t] * gC);
    // output: Y = gamma o (Q S) + P E
    f32x4 Yt[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) Yt[rt] = mma_f16(pf[rt], eb, G4[rt] * QS[rt]);
    const int64_t t0 = bos + static_cast<int64_t>(x) * kC;
    const int valid = static_cast<int>(len - static_cast<int64_t>(x) * kC < kC
                                           ? len - static_cast<int64_t>(x) * kC
                                           : kC);
    TOUT *yp = y + static_cast<size_t>(t0 * H + h) * DV + v0 + slab + lc;
    const size_t rstride = static_cast<size_t>(H) * DV;
    if (valid == kC) {
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) store_out(yp + (16 * rt + 4 * lg + i) * rstride, Yt[rt][i]);
    } else {
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * rt + 4 * lg + i < valid) store_out(yp + (16 * rt + 4 * lg + i) * rstride, Yt[rt][i]);
    }
  };

  // ---- pipeline -------------------------------------------------------------
  if (!is_state && nc > 0) {
#pragma unroll 1
    for (int x = 0; x < kDepth; ++x) issue_chunk(x);
  }
  if (!is_state) {
    // chunk 0 must have landed before the prologue computes it
    if (is_p0) wait_vmcnt<(kDepth - 1) * L::LOADS_P0>();
    else wait_vmcnt<(kDepth - 1) * L::LOADS_P1>();
  }
  wg_barrier();
  if (nc > 0) {
    if (is_p0) prep0(0);
    else if (!is_state) prep1(0);
  }
  if (!is_state) {
    if (is_p0) wait_vmcnt<(kDepth - 2) * L::LOADS_P0>();
    else wait_vmcnt<(kDepth - 2) * L::LOADS_P1>();
  }
  wg_barrier();
#pragma unroll 1
  for (int x = 0; x < nc; ++x) {
    if (is_state) {
      state_step(x);
    } else {
      issue_chunk(x + kDepth);
      if (x + 1 < nc) {
        if (is_p0) prep0(x + 1);
        else prep1(x + 1);
      }
      if (is_p0) wait_vmcnt<(kDepth - 2) * L::LOADS_P0>();
      else wait_vmcnt<(kDepth - 2) * L::LOADS_P1>();
    }
    wg_barrier();
  }
  if (!is_state) wait_vmcnt<0>();  // drain before the workgroup retires

  if (is_state && S_T) {
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_T[sbase + static_cast<size_t>(state_row(t, lg, i)) * DV] = st[t][i];
  }
}

template <int DK, int NS, typename TIN, typename TOUT>
hipError_t launch_bf16(const ChunkArgs &a) {
  constexpr int DVT = 16 * NS;
  const int n_vt = a.dv / DVT;
  const int64_t units = static_cast<int64_t>(a.N) * a.H;
  const int64_t blocks = (units + 7) / 8 * 8 * n_vt;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_fwd_bf16_kernel<DK, NS, TIN, TOUT>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * (NS + 2)), 0, a.stream, static_cast<const TIN *>(a.q),
                     static_cast<const TIN *>(a.k), static_cast<const TIN *>(a.v),
                     a.log_alpha, a.beta, a.S0, static_cast<TOUT *>(a.y), a.S_T, a.cu_seqlens,
                     a.T, a.H, a.dv, n_vt, static_cast<int>(units));
  return hipGetLastError();
}

}  // namespace

template <typename TIN, typename TOUT>
static hipError_t launch_16(const ChunkArgs &a) {
  return a.dk == 128 ? launch_bf16<128, 2, TIN, TOUT>(a) : launch_bf16<64, 2, TIN, TOUT>(a);
}

template <typename TIN>
static hipError_t launch_16_out(const ChunkArgs &a) {
  switch (a.out_dtype) {
    case 1: return launch_16<TIN, bf16_t>(a);
    case 2: return launch_16<TIN, _Float16>(a);
    default: return launch_16<TIN, float>(a);
  }
}

hipError_t launch_chunk_fwd_bf16(const ChunkArgs &a) {
  return a.in_dtype == 2 ? launch_16_out<_Float16>(a) : launch_16_out<bf16_t>(a);
}

hipError_t launch_chunk_fwd(const ChunkArgs &a) {
  return a.in_dtype == 0 ? launch_chunk_fwd_f32(a) : launch_chunk_fwd_bf16(a);
}

}  // namespace gdn
