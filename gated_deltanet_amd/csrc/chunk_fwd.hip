// Chunked parallel prefill of the gated delta rule, 16-bit inputs (gfx950).
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
// the state) and walks the sequence's chunks in order. Its NS "state" waves
// keep their 16-column slabs of the fp32 state in registers for the whole
// sequence and run the serial part: X = K S (bf16 MFMA, A operands straight
// from the raw K tile), Q S (fp16 MFMA on queries widened to fp16 in their
// registers), R, E = T R, Y = gamma QS + P E and the state update (fp16 MFMA).
// Four "prep" waves produce everything that does not depend on the state,
// pipelined ahead of the state waves:
//   * gram    (two chunks ahead): the Gram tiles K K^T on MFMA and A;
//   * inverse (one chunk ahead): T = (I + A)^{-1}: 16x16 diagonal blocks by
//             forward substitution in fp32, the off-diagonal block on MFMA;
//   * qk      (one chunk ahead): P = tril(Q K^T o G) computed as K Q^T so
//             that the MFMA result already sits in P's operand layout;
//   * kt      (one chunk ahead): half of the Kt^T tiles, transposed on the
//             matrix cores with a 0/1 selector operand (exact) and scaled
//             per token.
// Two more waves issue the direct-to-LDS loads (buffer_load ... lds) of K and
// the gates, and of Q and V, into a ring of LDS slots and wait for them:
// issuing those loads stalls the issuing wave for hundreds of cycles per
// chunk, which the compute waves no longer pay. Their spare time goes to the
// gate scan (wavefront prefix sum) and decay factors of the chunk just
// loaded, and to the other half of the Kt^T tiles. The loads go through
// buffer resources that end at the sequence's last row, so rows past the end
// read as zeros and no per-row clamping is needed. One workgroup barrier per
// chunk step hands finished chunks from stage to stage.
//
// Operand layouts in LDS are "fragment-linear": a 16x32 MFMA operand slice is
// stored as 64 lanes x 16 bytes, lane L's eight values contiguous at 16*L, so
// every operand read is one conflict-free ds_read_b128. To make the raw K/Q
// rows land that way straight from HBM, the key dimension inside each
// 32-slice is visited in the order 8*lg + j for lane group lg and slot j, and
// the state rows are stored in the matching order (see state_row()). With two
// state waves the raw K and Q tiles are instead kept in blocks of 8 tokens,
// so that each load fetches whole cache lines; their fragment reads are still
// one ds_read_b128 per lane at a per-lane base plus a constant (see frag()).
#include <cstdlib>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 32;     // tokens per chunk
constexpr int kNCT = 2;    // 16-token tiles per chunk
constexpr int kPrep = 6;   // prep waves per workgroup (four compute, two load)
constexpr int kLptMax = 256;  // packed batches up to this many sequences are run longest first

// LDS layout (bytes) for key size DK and NS state waves.
template <int DK, int NS>
struct Lay {
  static constexpr int DVT = 16 * NS;
  static constexpr int NKB = DK / 32;  // 32-deep key slices
  static constexpr int NST = DK / 16;  // 16-row state tiles
  // ring slot: raw 16-bit tiles of one chunk, loaded straight from HBM
  static constexpr int K_OFF = 0;
  static constexpr int Q_OFF = K_OFF + kNCT * NKB * 1024;
  static constexpr int V_OFF = Q_OFF + kNCT * NKB * 1024;
  static constexpr int G_OFF = V_OFF + kC * DVT * 2;  // log_alpha[32], beta[32]
  static constexpr int SLOT = G_OFF + 256;
  // raw-tile ring slots: six with one or two state waves, five with four
  // and four with eight (wider V tiles)
  static constexpr int RING_N = NS <= 2 ? 6 : NS == 4 ? 5 : 4;
  // per-chunk gate values (four buffers), 32 floats each:
  //   G2 running log2 decay, BT beta, GAM gamma = 2^G2, RA 2^(G2 - G2[m]),
  //   CB 2^(G2[m] - G2), KD 2^(G2[C-1] - G2), BR beta * RA, MISC[0] fast flag
  static constexpr int GB_G2 = 0, GB_BT = 128, GB_GAM = 256, GB_RA = 384, GB_CB = 512,
                       GB_KD = 640, GB_BR = 768, GB_MISC = 896;
  static constexpr int GATE = 1024;
  // processed operands (double-buffered): T, P, Kt^T fragments
  static constexpr int T_OFF = 0;
  static constexpr int P_OFF = T_OFF + kNCT * 1024;
  static constexpr int KT_OFF = P_OFF + kNCT * 1024;
  static constexpr int PROC = KT_OFF + NST * 1024;
  // fp32 A^T (double-buffered) and the inverse wave's scratch for T
  static constexpr int LDA = kC + 4;  // A^T row stride (floats)
  static constexpr int LDT = kC + 4;  // T row stride (floats), rows 16-byte aligned
  static constexpr int AMTB = kC * LDA * 4;
  static constexpr int RING = 0;
  static constexpr int PROCB = RING + RING_N * SLOT;
  static constexpr int GATEB = PROCB + 2 * PROC;
  static constexpr int AMT = GATEB + 4 * GATE;
  static constexpr int TMP = AMT + 2 * AMTB;
  static constexpr int TOTAL = TMP + kC * LDT * 4;
  // direct-to-LDS loads per chunk issued by the gram and qk waves
  static constexpr int NV = kC * DVT * 2 / 1024;    // V tile, 1 KiB per load
  static constexpr int LOADS_GRAM = kNCT * NKB + 2;  // K, log_alpha, beta
  static constexpr int LOADS_QK = kNCT * NKB + NV;   // Q, V
  static_assert(kC * DVT * 2 % 1024 == 0, "V tile must be whole KiB");
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  // generic -> LDS address-space conversion yields the 32-bit LDS offset
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char *)(p)));
}

// Raw buffer resource over [base, base + bytes): loads at or past the end
// return zeros, stores there are dropped.
__device__ __forceinline__ i32x4 buffer_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = static_cast<int32_t>(static_cast<uint32_t>(a));
  r[1] = static_cast<int32_t>(static_cast<uint32_t>(a >> 32));  // stride 0
  r[2] = static_cast<int32_t>(bytes);
  r[3] = 0x00020000;  // raw dword access
  return r;
}

// Direct-to-LDS loads: lane L's data lands at (M0 + 16*L) or (M0 + 4*L).
// Written in asm so the compiler does not serialise later LDS reads behind
// them; completion is tracked explicitly with vmcnt waits. M0 is written one
// wait state before the load reads it.
__device__ __forceinline__ void dma16(const i32x4 &rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               ::"v"(voff), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const i32x4 &rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               ::"v"(voff), "s"(rsrc), "s"(lds)
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
// y element stores through a buffer resource (rows past its end are dropped)
template <typename TOUT>
__device__ __forceinline__ void store_y(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (std::is_same<TOUT, float>::value)
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r,
                                          static_cast<int>(off), 0, 0);
  else if constexpr (std::is_same<TOUT, bf16_t>::value)
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)v), r,
                                          static_cast<int>(off), 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)v), r,
                                          static_cast<int>(off), 0, 0);
}

// Operations on the raw 16-bit input tiles (K, Q, V) for each input type.
// bf16 inputs keep bf16 operands for the key-side products (exact inputs;
// the state operand of K S is rounded to bf16) and have Q widened to fp16 in
// the state waves' registers for Q S; fp16 inputs use fp16 operands throughout.
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

// STATES: write every chunk-start state, in fp16, to `states` (the backward pass's
// workspace) instead of y and S_T. LPT (packed batches of at most kLptMax
// sequences): workgroups take the sequences longest first, so the short ones
// fill in at the end instead of a long one running alone.
template <int DK, int NS, typename TIN, typename TOUT, bool STATES, bool LPT, bool SEG>
__global__ __launch_bounds__(64 * (NS + kPrep)) void chunk_fwd_bf16_kernel(
    const TIN *__restrict__ q, const TIN *__restrict__ k, const TIN *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    const float *__restrict__ gA, const float *__restrict__ gbias,
    const float *__restrict__ S0, TOUT *__restrict__ y, float *__restrict__ S_T,
    float *__restrict__ states, const int32_t *__restrict__ cu_seqlens, int T, int H, int DV,
    int n_vt, int n_units, SegCtl seg) {
  using L = Lay<DK, NS>;
  using KO = KOps<TIN>;
  using kvec = typename KO::vec;
  constexpr int NKB = L::NKB;
  constexpr int NST = L::NST;
  constexpr int DVT = L::DVT;
  constexpr int NTHR = 64 * (NS + kPrep);
  constexpr int kRing = L::RING_N;
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
  int n = unit / H;
  if constexpr (LPT) {
    // dispatch position n takes the sequence of rank n by length (longest
    // first, ties by index); every workgroup ranks the lengths itself, in the
    // LDS before it is cleared
    int *lens = reinterpret_cast<int *>(smem);
    int *pick = lens + kLptMax;
    const int N = units / H;
    for (int j = threadIdx.x; j < N; j += NTHR) {
      int64_t a = cu_seqlens[j], b = cu_seqlens[j + 1];
      a = a < 0 ? 0 : (a > T ? T : a);
      b = b < a ? a : (b > T ? T : b);
      lens[j] = static_cast<int>(b - a);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < N; j += NTHR) {
      const int lj = lens[j];
      int rank = 0;
      for (int m = 0; m < N; ++m) {
        const int lm = lens[m];
        rank += (lm > lj) || (lm == lj && m < j);
      }
      if (rank == n) *pick = j;
    }
    __syncthreads();
    n = *pick;
    __syncthreads();
  }
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
  // the controls of the segment runs are read only by the SEG variant, so
  // that every other instantiation compiles as if they were absent
  const bool write_y = !SEG || (y != nullptr && n < seg.y_nseq);  // (never for the states-only variant)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int v0 = vt * DVT;
  // Layout of the raw K and Q tiles in the ring. With two state waves
  // (kRowBlocks) a tile is stored in 1 KiB blocks of 8 tokens x 64 keys, so
  // that each direct-to-LDS load fetches 8 whole 128-byte lines (8 rows, half
  // a row each at d = 128) instead of 16 half lines: lane L of a block holds
  // row L % 8, keys 8 (L / 8) .. 8 (L / 8) + 7. Otherwise each 1 KiB block is
  // one 16 x 32 MFMA operand slice, lane L's 16 bytes at 16 L. Either way the
  // 16 bytes lane (lg, lc) reads for row tile rt and 32-key slice kb (row
  // 16 rt + lc, keys 32 kb + 8 lg .. 32 kb + 8 lg + 7) sit at a per-lane base
  // plus a constant per (rt, kb), so the operand reads need no per-slice
  // address arithmetic, and 8 consecutive lanes read distinct banks. (With
  // one state wave the eight column tiles of a head then shared their K and Q
  // reads less well in L2: 35% more HBM reads on B1 H32 T65536.)
  constexpr bool kRowBlocks = NS == 2;
  constexpr int kHalves = DK / 64;  // 64-key halves per row
  int frag_lane = kRowBlocks ? 1024 * kHalves * (lc >> 3) + 128 * lg + 16 * (lc & 7) : 0;
  if constexpr (kRowBlocks)
    asm volatile("" : "+v"(frag_lane));  // opaque: kept apart from the other per-lane offsets
  auto frag = [&](int rt, int kb) -> int {
    if constexpr (kRowBlocks)
      return frag_lane + 1024 * (2 * kHalves * rt + (kb >> 1)) + 512 * (kb & 1);
    else
      return (rt * NKB + kb) * 1024 + 16 * lane;
  };
  // roles; wave w runs on SIMD w % 4, so the two helpers that share a SIMD
  // with a state wave (gram, kt) are the lighter ones
  const bool is_state = wave < NS;
  const bool is_inv = wave == NS;
  const bool is_qk = wave == NS + 1;
  const bool is_gram = wave == NS + 2;  // wave NS + 3: kt
  const bool is_ldk = wave == NS + 4;   // loads K and the gates
  const bool is_ldq = wave == NS + 5;   // loads Q and V
  const int slab = 16 * wave;  // state waves: first column of the slab

  char *const ring = smem + L::RING;
  char *const procb = smem + L::PROCB;
  char *const gateb = smem + L::GATEB;
  float *const tmp = reinterpret_cast<float *>(smem + L::TMP);
  auto amt_of = [&](int c) { return reinterpret_cast<float *>(smem + L::AMT + (c & 1) * L::AMTB); };
  auto gate_of = [&](int c) {
    return reinterpret_cast<float *>(gateb + (c & 3) * L::GATE);
  };

  // Zero all of LDS once: the parts of the operand buffers that are never
  // written (upper blocks of T and P) must read as zeros, and ring rows that
  // a chunk past the end of the sequence does not load hold finite values.
  for (int i = threadIdx.x; i < L::TOTAL / 16; i += NTHR)
    reinterpret_cast<f32x4 *>(smem)[i] = zero4();
  wg_barrier();

  // ---- direct-to-LDS loads of chunk c into its ring slot --------------------
  // The buffer resource of each tensor starts at the chunk's first row and
  // ends after its last row inside the sequence, so rows past the end read as
  // zeros; per-lane offsets are fixed for the whole sequence.
  const int hdk = H * DK;
  const int hdv = H * DV;
  auto rows_of = [&](int c) -> int {
    const int64_t r = len - static_cast<int64_t>(c) * kC;
    return r <= 0 ? 0 : (r >= kC ? kC : static_cast<int>(r));
  };
  auto row0_of = [&](int c) -> int64_t {
    const int64_t r = static_cast<int64_t>(c) * kC;
    return bos + (r < len ? r : len);
  };
  // per-lane byte offsets of this lane's K/Q and V pieces inside a chunk:
  // load j of a K or Q tile fills block j of the tile (the layout above)
  const uint32_t kq_lane = static_cast<uint32_t>((lc * hdk + h * DK + 8 * lg) * 2);
  auto kq_load = [&](int j) -> uint32_t {
    if constexpr (kRowBlocks) {
      const int r = 8 * (j / kHalves) + (lane & 7);
      return static_cast<uint32_t>((r * hdk + h * DK) * 2 + 128 * (j % kHalves) + 16 * (lane >> 3));
    } else {
      return kq_lane + static_cast<uint32_t>(16 * (j / NKB) * hdk * 2 + 64 * (j % NKB));
    }
  };
  auto v_lane = [&](int p) -> uint32_t {
    const int qi = 64 * p + lane;
    const int r = qi / (DVT / 8);
    const int cc = qi % (DVT / 8);
    return static_cast<uint32_t>((r * hdv + h * DV + v0 + 8 * cc) * 2);
  };
  const uint32_t g_off = static_cast<uint32_t>(((lane & 31) * H + h) * 4);

  auto issue_gram = [&](int c) {
    char *slot = ring + (c % kRing) * L::SLOT;
    const int64_t r0 = row0_of(c);
    const uint32_t rows = static_cast<uint32_t>(rows_of(c));
    const i32x4 rk = buffer_rsrc(k + r0 * hdk, rows * hdk * 2);
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        dma16(rk, kq_load(rt * NKB + kb), lds_addr(slot + L::K_OFF + (rt * NKB + kb) * 1024));
    const i32x4 rla = buffer_rsrc(log_alpha + r0 * H, rows * H * 4);
    const i32x4 rb = buffer_rsrc(beta + r0 * H, rows * H * 4);
    if (lane < 32) dma4(rla, g_off, lds_addr(slot + L::G_OFF));
    else dma4(rb, g_off, lds_addr(slot + L::G_OFF));
  };
  auto issue_qk = [&](int c) {
    char *slot = ring + (c % kRing) * L::SLOT;
    const int64_t r0 = row0_of(c);
    const uint32_t rows = static_cast<uint32_t>(rows_of(c));
    const uint32_t vrows = SEG && seg.v_zero ? 0u : rows;  // v read as zeros: an empty range
    if constexpr (!STATES) {  // the states-only variant never reads Q
      // Q only feeds y: a run that writes no y loads it from an empty range
      const i32x4 rq = buffer_rsrc(q + r0 * hdk, (write_y ? rows : 0u) * hdk * 2);
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          dma16(rq, kq_load(rt * NKB + kb), lds_addr(slot + L::Q_OFF + (rt * NKB + kb) * 1024));
    }
    const i32x4 rv = buffer_rsrc(v + r0 * hdv, vrows * hdv * 2);
#pragma unroll
    for (int p = 0; p < L::NV; ++p) dma16(rv, v_lane(p), lds_addr(slot + L::V_OFF + p * 1024));
  };

  // ---- gram wave: gate scan, decay factors, Gram tiles, A ------------------
  // Running sums are kept in log2 units (g2 = g / ln 2) so every decay is a
  // single v_exp_f32. Within a chunk the decay G_rc = 2^(g2_r - g2_c) factors
  // as a_r * b_c with a_r = 2^(g2_r - g2_m), b_c = 2^(g2_m - g2_c) around the
  // middle token m; that replaces one exponential per matrix element by one
  // per row. The factorisation is used only when both factors stay well
  // inside the fp32 range; otherwise (extreme gates) the chunk falls back to
  // one exponential per element. The branch is uniform per chunk.
  const RawGate gate = RawGate::load(gA, gbias, h);
  auto scan_gates = [&](int c) {
    const char *slot = ring + (c % kRing) * L::SLOT;
    float *gt = gate_of(c);
    const float *gl = reinterpret_cast<const float *>(slot + L::G_OFF);
    const int64_t tok = static_cast<int64_t>(c) * kC + lane;
    float la = 0.0f, bt = 0.0f;
    if (lane < kC && tok < len) {
      la = gl[lane];
      bt = gl[32 + lane];
      if (gate.raw()) {
        la = gate.log_alpha(la);
        bt = RawGate::beta(bt);
      }
    }
    float sc = la * 1.4426950408889634f;
    sc += dpp_shr<1>(sc);
    sc += dpp_shr<2>(sc);
    sc += dpp_shr<4>(sc);
    sc += dpp_shr<8>(sc);
    const float r15 = readlane(sc, 15);
    if (lane >= 16) sc += r15;
    const float gC2 = readlane(sc, kC - 1);
    const float gm2 = r15;
    const float g0 = readlane(sc, 0);
    const bool fast = (g0 - gm2 <= 120.0f) && (gm2 - gC2 <= 120.0f);
    const float ra = __builtin_amdgcn_exp2f(sc - gm2);
    if (lane < kC) {
      gt[L::GB_G2 / 4 + lane] = sc;
      gt[L::GB_BT / 4 + lane] = bt;
      gt[L::GB_GAM / 4 + lane] = __builtin_amdgcn_exp2f(sc);
      gt[L::GB_RA / 4 + lane] = ra;
      gt[L::GB_CB / 4 + lane] = __builtin_amdgcn_exp2f(gm2 - sc);
      gt[L::GB_KD / 4 + lane] = __builtin_amdgcn_exp2f(gC2 - sc);
      gt[L::GB_BR / 4 + lane] = bt * ra;
    }
    if (lane == 0) gt[L::GB_MISC / 4] = fast ? 1.0f : 0.0f;
  };
  auto gram = [&](int c) {
    const char *slot = ring + (c % kRing) * L::SLOT;
    const float *gt = gate_of(c);
    kvec kf[kNCT][NKB];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        kf[rt][kb] = lds_read16<kvec>(slot + L::K_OFF + frag(rt, kb));
    const bool fast = __builtin_amdgcn_readfirstlane(
                          __builtin_bit_cast(int, gt[L::GB_MISC / 4])) != 0;
    f32x4 gm[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) gm[t] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      gm[0] = KO::mma(kf[0][kb], kf[0][kb], gm[0]);
      gm[1] = KO::mma(kf[1][kb], kf[0][kb], gm[1]);
      gm[2] = KO::mma(kf[1][kb], kf[1][kb], gm[2]);
    }
    // A = strictly_lower(diag(beta) (K K^T o G)); tile t = (row tile, col tile)
    // (0,0), (1,0), (1,1); element i of lane (lg, lc) is row 4 lg + i, column lc
    f32x4 av[3];
    if (fast) {
      f32x4 br[kNCT];
      float cb[kNCT];
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt) {
        br[rt] = *reinterpret_cast<const f32x4 *>(gt + L::GB_BR / 4 + 16 * rt + 4 * lg);
        cb[rt] = gt[L::GB_CB / 4 + 16 * rt + lc];
      }
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int rt = t == 0 ? 0 : 1, ct = t == 2 ? 1 : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) av[t][i] = br[rt][i] * cb[ct] * gm[t][i];
      }
    } else {
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int rt = t == 0 ? 0 : 1, ct = t == 2 ? 1 : 0;
        const f32x4 gr = *reinterpret_cast<const f32x4 *>(gt + L::GB_G2 / 4 + 16 * rt + 4 * lg);
        const f32x4 bv = *reinterpret_cast<const f32x4 *>(gt + L::GB_BT / 4 + 16 * rt + 4 * lg);
        const float gc = gt[L::GB_G2 / 4 + 16 * ct + lc];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[t][i] = bv[i] * __builtin_amdgcn_exp2f(fminf(gr[i] - gc, 0.0f)) * gm[t][i];
      }
    }
    // stored transposed (A^T row c = column c of A) in fp32
    float *amt = amt_of(c);
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int rt = t == 0 ? 0 : 1, ct = t == 2 ? 1 : 0;
      const int col = 16 * ct + lc;
      f32x4 a;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = (16 * rt + 4 * lg + i > col) ? av[t][i] : 0.0f;
      *reinterpret_cast<f32x4 *>(amt + col * L::LDA + 16 * rt + 4 * lg) = a;
    }
  };

  // ---- inverse wave: T = (I + A)^{-1} ----------------------------------------
  auto inverse = [&](int c) {
    const float *amt = amt_of(c);
    char *pb = procb + (c & 1) * L::PROC;
    // A_10 in the layout of an MFMA A operand, read ahead of the solve:
    // slot j of lane (lg, lc) is A[16 + lc][4 lg + j] (A is stored transposed)
    float a10[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a10[j] = amt[(4 * lg + j) * L::LDA + 16 + lc];
    // Diagonal 16x16 blocks by forward substitution. Each 16-lane row works
    // on one block (rows 2 and 3 repeat rows 0 and 1); lane lc holds column lc
    // of T and column lc of A, so A is read from LDS once (unit_lower_solve16).
    {
      const int b = lg & (kNCT - 1);
      float ac[16], xv[16];
      const float *acol = amt + (16 * b + lc) * L::LDA + 16 * b;  // A[16b + r][16b + lc]
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 t4 = *reinterpret_cast<const f32x4 *>(acol + 4 * u);
#pragma unroll
        for (int i = 0; i < 4; ++i) ac[4 * u + i] = t4[i];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) xv[r] = (r == lc) ? 1.0f : 0.0f;
      unit_lower_solve16(ac, xv);

      if (lg < kNCT) {
#pragma unroll
        for (int r = 0; r < 16; ++r) tmp[(16 * b + r) * L::LDT + 16 * b + lc] = xv[r];
      }
    }
    wait_lds();
    // off-diagonal block: T_10 = -T_11 (A_10 T_00). The second product is
    // formed with its operands swapped, which yields (T_11 M)^T: lane (lg, lc)
    // then holds T_10[lc][4 lg + i], the row layout T is stored in, so T_10
    // goes straight from the matrix core into the T fragments.
    {
      f16x8 a, bb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = (_Float16)a10[j];
        bb[j] = (_Float16)tmp[(4 * lg + j) * L::LDT + lc];  // T_00[4 lg + j][lc]
        a[4 + j] = (_Float16)0.0f;
        bb[4 + j] = (_Float16)0.0f;
      }
      const f32x4 t00r = *reinterpret_cast<const f32x4 *>(tmp + lc * L::LDT + 4 * lg);
      const f32x4 t11r = *reinterpret_cast<const f32x4 *>(tmp + (16 + lc) * L::LDT + 16 + 4 * lg);
      const f32x4 M = mma_f16(a, bb, zero4());  // M[4 lg + i][lc] = (A_10 T_00)
      f16x8 mb, t11;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mb[j] = (_Float16)M[j];      // M^T as the A operand
        t11[j] = (_Float16)t11r[j];  // T_11^T as the B operand: T_11[lc][4 lg + j]
        mb[4 + j] = (_Float16)0.0f;
        t11[4 + j] = (_Float16)0.0f;
      }
      const f32x4 D = mma_f16(mb, t11, zero4());
      // T in fragment-linear fp16: row 16 mt + lc, slot j <-> token
      // 16 (j >> 2) + 4 lg + (j & 3); the upper right block is zero
      *reinterpret_cast<f16x8 *>(pb + L::T_OFF + 16 * lane) = pack_f16(t00r, zero4());
      *reinterpret_cast<f16x8 *>(pb + L::T_OFF + 1024 + 16 * lane) = pack_f16(-D, t11r);
    }
  };

  // 0/1 selector operand for exact transposes on the matrix cores: in lane
  // (lg, lc), slot j is 1 iff lg == lc >> 2 and j == 4u + (lc & 3).
  auto selector = [&](int u) {
    kvec s_;
#pragma unroll
    for (int j = 0; j < 8; ++j) s_[j] = (lg == (lc >> 2) && j == 4 * u + (lc & 3)) ? 1.0f : 0.0f;
    return s_;
  };

  // ---- qk wave: P = tril(Q K^T o G) -----------------------------------------
  auto qkp = [&](int c) {
    const char *slot = ring + (c % kRing) * L::SLOT;
    char *pb = procb + (c & 1) * L::PROC;
    const float *gt = gate_of(c);
    kvec kf[kNCT][NKB], qf[kNCT][NKB];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        kf[rt][kb] = lds_read16<kvec>(slot + L::K_OFF + frag(rt, kb));
        qf[rt][kb] = lds_read16<kvec>(slot + L::Q_OFF + frag(rt, kb));
      }
    const bool fast = __builtin_amdgcn_readfirstlane(
                          __builtin_bit_cast(int, gt[L::GB_MISC / 4])) != 0;
    // decay factors of both forms, read up front with the operands so that
    // their latency overlaps the products
    float ar[kNCT], gr[kNCT];
    f32x4 cb[kNCT], gc[kNCT];
#pragma unroll
    for (int t = 0; t < kNCT; ++t) {
      ar[t] = gt[L::GB_RA / 4 + 16 * t + lc];
      cb[t] = *reinterpret_cast<const f32x4 *>(gt + L::GB_CB / 4 + 16 * t + 4 * lg);
      gr[t] = gt[L::GB_G2 / 4 + 16 * t + lc];
      gc[t] = *reinterpret_cast<const f32x4 *>(gt + L::GB_G2 / 4 + 16 * t + 4 * lg);
    }
    // K Q^T: element i of lane (lg, lc) in tile (ct, rt) is P[16 rt + lc][16 ct + 4 lg + i],
    // i.e. slot i (ct = 0) or 4 + i (ct = 1) of P's operand fragment for row tile rt
    f32x4 pk[3];  // (ct, rt) = (0, 0), (0, 1), (1, 1)
#pragma unroll
    for (int t = 0; t < 3; ++t) pk[t] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      pk[0] = KO::mma(kf[0][kb], qf[0][kb], pk[0]);
      pk[1] = KO::mma(kf[0][kb], qf[1][kb], pk[1]);
      pk[2] = KO::mma(kf[1][kb], qf[1][kb], pk[2]);
    }
    f32x4 pv[3];
    if (fast) {
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int ct = t == 2 ? 1 : 0, rt = t == 0 ? 0 : 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[t][i] = ar[rt] * cb[ct][i] * pk[t][i];
      }
    } else {
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int ct = t == 2 ? 1 : 0, rt = t == 0 ? 0 : 1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pv[t][i] = __builtin_amdgcn_exp2f(fminf(gr[rt] - gc[ct][i], 0.0f)) * pk[t][i];
      }
    }
    // causal mask on the diagonal tiles: column 4 lg + i <= row lc
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[0][i] = (4 * lg + i <= lc) ? pv[0][i] : 0.0f;
      pv[2][i] = (4 * lg + i <= lc) ? pv[2][i] : 0.0f;
    }
    *reinterpret_cast<f16x8 *>(pb + L::P_OFF + 16 * lane) = pack_f16(pv[0], zero4());
    *reinterpret_cast<f16x8 *>(pb + L::P_OFF + 1024 + 16 * lane) = pack_f16(pv[1], pv[2]);
  };

  // ---- kt wave: Kt^T ---------------------------------------------------------
  // For each state tile, transpose 16 keys x 32 tokens on the matrix cores
  // and scale token columns by exp(g_C - g_t).
  auto ktt = [&](int c, int half) {
    const char *slot = ring + (c % kRing) * L::SLOT;
    char *pb = procb + (c & 1) * L::PROC;
    const float *gt = gate_of(c);
    kvec kf[kNCT][NKB];  // only the key slices of this half's state tiles are read
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
      for (int kb = half * (NKB / 2); kb < (half + 1) * (NKB / 2); ++kb)
        kf[rt][kb] = lds_read16<kvec>(slot + L::K_OFF + frag(rt, kb));
    const kvec sel[2] = {selector(0), selector(1)};
    // slot j of the A operand <-> token 16 (j >> 2) + 4 lg + (j & 3)
    const f32x4 kd0 = *reinterpret_cast<const f32x4 *>(gt + L::GB_KD / 4 + 4 * lg);
    const f32x4 kd1 = *reinterpret_cast<const f32x4 *>(gt + L::GB_KD / 4 + 16 + 4 * lg);
#pragma unroll
    for (int tt = 0; tt < NST / 2; ++tt) {
      const int t = half * (NST / 2) + tt;
      const f32x4 d0 = KO::mma(kf[0][t >> 1], sel[t & 1], zero4());
      const f32x4 d1 = KO::mma(kf[1][t >> 1], sel[t & 1], zero4());
      *reinterpret_cast<f16x8 *>(pb + L::KT_OFF + t * 1024 + 16 * lane) =
          pack_f16(kd0 * d0, kd1 * d1);
    }
  };

  // ---- state waves -----------------------------------------------------------
  f32x4 st[NST];
  const size_t sbase = static_cast<size_t>(n * H + h) * DK * DV + v0 + slab + lc;
  if (is_state) {
    __builtin_amdgcn_s_setprio(1);
    const bool use_s0 = S0 != nullptr && (!SEG || n < seg.s0_nseq);
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = state_row(t, lg, i);
        st[t][i] = SEG && seg.s0_ident ? (row == v0 + slab + lc ? 1.0f : 0.0f)
                   : use_s0            ? S0[sbase + static_cast<size_t>(row) * DV]
                                       : 0.0f;
      }
  }

  // chunk-start states for the backward pass (optional): chunk x of sequence
  // n goes to slot floor(bos / C) + n + x, in fp16 (the backward's 16-bit
  // products round the state to fp16 anyway), in blocks of 32 columns (the
  // backward's column tiles) of two 16-column slabs each
  _Float16 *const st_out =
      STATES ? reinterpret_cast<_Float16 *>(states) +
                   ((static_cast<size_t>(bos / kC + n) * H + h) * (DV / 32) + (v0 + slab) / 32) *
                       DK * 32 +
                   (static_cast<size_t>((v0 + slab) / 16 % 2) * NST * 64 + lane) * 4
             : nullptr;
  // byte offset of this lane's first y element inside a chunk's rows
  const uint32_t y_lane =
      static_cast<uint32_t>((4 * lg * hdv + h * DV + v0 + slab + lc) * sizeof(TOUT));

  // One chunk of the state waves. WITH_Y false (segment runs that write no
  // y: summaries and transitions) keeps only the chain X = K S -> R ->
  // E = T R -> S update and leaves out Q S, P E and the y stores.
  auto state_step = [&](int x, auto with_y) {
    constexpr bool WITH_Y = decltype(with_y)::value;
    if constexpr (STATES) {
      typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
      _Float16 *dst = st_out + static_cast<size_t>(x) * H * DK * DV;
#pragma unroll
      for (int t = 0; t < NST; ++t) {
        f16x4 h4;
#pragma unroll
        for (int i = 0; i < 4; ++i) h4[i] = static_cast<_Float16>(st[t][i]);
        *reinterpret_cast<f16x4 *>(dst + t * 256) = h4;
      }
    }
    const char *slot = ring + (x % kRing) * L::SLOT;
    const char *pb = procb + (x & 1) * L::PROC;
    const float *gt = gate_of(x);
    // every LDS operand of this chunk, issued up front
    kvec kf[kNCT][NKB];
    f16x8 qf[kNCT][NKB], tf[kNCT], pf[kNCT], ktf[NST];
    f32x4 G4[kNCT], B4[kNCT];
    uint16_t vraw[kNCT][4];
    const uint16_t *vt_ = reinterpret_cast<const uint16_t *>(slot + L::V_OFF);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt)
        kf[rt][kb] = lds_read16<kvec>(slot + L::K_OFF + frag(rt, kb));
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) {
      G4[rt] = *reinterpret_cast<const f32x4 *>(gt + L::GB_GAM / 4 + 16 * rt + 4 * lg);
      B4[rt] = *reinterpret_cast<const f32x4 *>(gt + L::GB_BT / 4 + 16 * rt + 4 * lg);
#pragma unroll
      for (int i = 0; i < 4; ++i) vraw[rt][i] = vt_[(16 * rt + 4 * lg + i) * DVT + slab + lc];
      tf[rt] = lds_read16<f16x8>(pb + L::T_OFF + rt * 1024 + 16 * lane);
    }
    const float gC = gt[L::GB_GAM / 4 + kC - 1];
#pragma unroll
    for (int t = 0; t < NST; ++t) ktf[t] = lds_read16<f16x8>(pb + L::KT_OFF + t * 1024 + 16 * lane);
    kvec qraw[kNCT][NKB];
    if constexpr (WITH_Y) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rt = 0; rt < kNCT; ++rt) {
          if constexpr (KO::kConvertQ)
            qraw[rt][kb] = lds_read16<kvec>(slot + L::Q_OFF + frag(rt, kb));
          else
            qf[rt][kb] = lds_read16<f16x8>(slot + L::Q_OFF + frag(rt, kb));
        }
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt) pf[rt] = lds_read16<f16x8>(pb + L::P_OFF + rt * 1024 + 16 * lane);
    }

    // the state as B operand: bf16 against the raw bf16 keys for X = K S,
    // fp16 against the fp16 queries for Q S (Q S feeds y directly, so it gets
    // the finer rounding; errors in X are largely corrected by the delta rule)
    kvec sb[NKB];
    f16x8 sh[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sb[kb] = KO::pack(st[2 * kb], st[2 * kb + 1]);
      if constexpr (WITH_Y) sh[kb] = pack_f16(st[2 * kb], st[2 * kb + 1]);
    }
    // serial chain: X = K S -> R -> E = T R -> S update. X is summed in two
    // halves so that no MFMA waits on the one just before it.
    f32x4 Xa[kNCT], Xb[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) {
      Xa[rt] = zero4();
      Xb[rt] = zero4();
    }
#pragma unroll
    for (int kb = 0; kb < NKB; kb += 2)
#pragma unroll
      for (int rt = 0; rt < kNCT; ++rt) {
        Xa[rt] = KO::mma(kf[rt][kb], sb[kb], Xa[rt]);
        Xb[rt] = KO::mma(kf[rt][kb + 1], sb[kb + 1], Xb[rt]);
      }
    // Q in fp16 for Q S (bf16 inputs): D_u = Sel_u x Q^T puts keys
    // 8 lg + 4u + i of token lc in lane (lg, lc), the A-operand slots the raw
    // tile already has, so the matrix cores only widen it (exact), and the
    // rounding to fp16 is exact for all but tiny values. Off the X -> R -> E
    // chain, so these products fill issue gaps of the state waves.
    if constexpr (WITH_Y && KO::kConvertQ) {
      const kvec sel[2] = {selector(0), selector(1)};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rt = 0; rt < kNCT; ++rt)
          qf[rt][kb] = pack_f16(KO::mma(sel[0], qraw[rt][kb], zero4()),
                                KO::mma(sel[1], qraw[rt][kb], zero4()));
    }
    f32x4 QS[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) QS[rt] = zero4();
    if constexpr (WITH_Y) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rt = 0; rt < kNCT; ++rt) QS[rt] = mma_f16(qf[rt][kb], sh[kb], QS[rt]);
    }
    f32x4 R[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        R[rt][i] = B4[rt][i] * fmaf(-G4[rt][i], Xb[rt][i],
                                    fmaf(-G4[rt][i], Xa[rt][i], KO::to_f32(vraw[rt][i])));
    const f16x8 rb = pack_f16(R[0], R[1]);
    f32x4 E[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) E[rt] = mma_f16(tf[rt], rb, zero4());
    const f16x8 eb = pack_f16(E[0], E[1]);
#pragma unroll
    for (int t = 0; t < NST; ++t) st[t] = mma_f16(ktf[t], eb, st[t] * gC);
    if constexpr (!WITH_Y) return;
    // output: Y = gamma o (Q S) + P E; rows past the end of the sequence fall
    // outside the buffer resource and are dropped
    f32x4 Yt[kNCT];
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt) Yt[rt] = mma_f16(pf[rt], eb, G4[rt] * QS[rt]);
    if (STATES || !write_y) return;
    const uint32_t rows = static_cast<uint32_t>(rows_of(x));
    const auto ry = __builtin_amdgcn_make_buffer_rsrc(y + row0_of(x) * hdv, 0,
                                                      static_cast<int>(rows * hdv * sizeof(TOUT)),
                                                      0x00020000);
#pragma unroll
    for (int rt = 0; rt < kNCT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) store_y<TOUT>(Yt[rt][i], ry,
                              y_lane + static_cast<uint32_t>((16 * rt + i) * hdv * sizeof(TOUT)));
  };

  // ---- pipeline -------------------------------------------------------------
  // Step it (it = -3 .. nc-1): the state waves run chunk it, the gram wave
  // chunk it + 2, the inverse, qk and kt waves chunk it + 1. The two load
  // waves: one issues K and the gates of chunk it + 3 + kLdK, waits for chunk
  // it + 3 (the gram wave's next chunk) and runs that chunk's gate scan; the
  // other issues Q and V of chunk it + 2 + kLdQ, builds half of the Kt^T
  // tiles of chunk it + 1 and waits for chunk it + 2 (the qk wave's next
  // chunk). A chunk's ring slot is reloaded only after the state waves have
  // finished it. Every role runs its own loop with one barrier per step
  // (nc + 3 in all).
  constexpr int kLdK = kRing - 4;
  constexpr int kLdQ = kRing - 3;
  constexpr int kLoadsQV = STATES ? L::NV : L::LOADS_QK;  // loads per chunk of the Q/V wave
  static_assert((kLdK + 1) * L::LOADS_GRAM < 64 && (kLdQ + 1) * kLoadsQV < 64, "vmcnt range");
  auto step_barrier = [&]() { wg_barrier(); };
  auto in_range = [&](int c) { return c >= 0 && c < nc; };
  if (nc > 0) {
    if (is_state) {
      step_barrier();
      step_barrier();
      step_barrier();
      if (SEG && !write_y) {
#pragma unroll 1
        for (int x = 0; x < nc; ++x) {
          state_step(x, std::false_type{});
          step_barrier();
        }
      } else {
#pragma unroll 1
        for (int x = 0; x < nc; ++x) {
          state_step(x, std::true_type{});
          step_barrier();
        }
      }
    } else if (is_ldk) {
#pragma unroll 1
      for (int c = 0; c < kLdK; ++c) issue_gram(c);
#pragma unroll 1
      for (int it = -3; it < nc; ++it) {
        issue_gram(it + 3 + kLdK);
        wait_vmcnt<kLdK * L::LOADS_GRAM>();
        if (in_range(it + 3)) scan_gates(it + 3);
        step_barrier();
      }
      wait_vmcnt<0>();  // drain before the workgroup retires
    } else if (is_ldq) {
#pragma unroll 1
      for (int c = 0; c < kLdQ - 1; ++c) issue_qk(c);
#pragma unroll 1
      for (int it = -3; it < nc; ++it) {
        issue_qk(it + 2 + kLdQ);
        if (in_range(it + 1)) ktt(it + 1, 1);
        wait_vmcnt<kLdQ * kLoadsQV>();
        step_barrier();
      }
      wait_vmcnt<0>();
    } else {
#pragma unroll 1
      for (int it = -3; it < nc; ++it) {
        if (is_gram) {
          if (in_range(it + 2)) gram(it + 2);
        } else if (is_qk) {
          if (!STATES && write_y && in_range(it + 1)) qkp(it + 1);  // P only feeds y
        } else if (is_inv) {
          if (in_range(it + 1)) inverse(it + 1);
        } else {
          if (in_range(it + 1)) ktt(it + 1, 0);
        }
        step_barrier();
      }
    }
  }

  const int st_first = SEG ? seg.st_first : 0;
  if (!STATES && is_state && S_T && n >= st_first) {
    const size_t obase = static_cast<size_t>((n - st_first) * H + h) * DK * DV + v0 + slab + lc;
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_T[obase + static_cast<size_t>(state_row(t, lg, i)) * DV] = st[t][i];
  }
}

template <int DK, int NS, typename TIN, typename TOUT, bool STATES = false, bool LPT = false,
          bool SEG = false>
hipError_t launch_bf16(const ChunkArgs &a) {
  constexpr int DVT = 16 * NS;
  const int n_vt = a.dv / DVT;
  const int64_t units = static_cast<int64_t>(a.N) * a.H;
  const int64_t blocks = (units + 7) / 8 * 8 * n_vt;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_fwd_bf16_kernel<DK, NS, TIN, TOUT, STATES, LPT, SEG>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * (NS + kPrep)), 0, a.stream, static_cast<const TIN *>(a.q),
                     static_cast<const TIN *>(a.k), static_cast<const TIN *>(a.v),
                     a.log_alpha, a.beta, a.A, a.b_alpha, a.S0, static_cast<TOUT *>(a.y), a.S_T, a.states, a.cu_seqlens,
                     a.T, a.H, a.dv, n_vt, static_cast<int>(units), a.seg);
  return hipGetLastError();
}

}  // namespace

// State waves per workgroup. Each column tile of a head repeats the head's
// prep work (gate scan, Gram, inverse, Q K^T), so wider tiles do less work
// in all but take longer per step (more waves share the SIMDs) and give
// fewer workgroups. With one workgroup per CU the time is about (rounds of
// workgroups) x (step time); relative step times measured on the varlen
// front-end and the B4 H16 T4096 / B1 H32 T65536 workloads: 1 wave 0.92,
// 2 waves 1, 4 waves 1.29, 8 waves 2.06. The count with the least estimate
// is taken (ties to fewer waves). GDN_PREFILL_NS = 1, 2, 4 or 8 sets it
// instead (a test hook).
static int prefill_ns(const ChunkArgs &a) {
  if (a.dk != 128 || a.dv % 64 != 0) return 2;
  if (const char *e = getenv("GDN_PREFILL_NS")) {
    const int ns = atoi(e);
    if (ns == 1 || ns == 2 || ns == 4 || (ns == 8 && a.dv % 128 == 0)) return ns;
  }
  constexpr int64_t kCUs = 256;
  const int64_t slabs = static_cast<int64_t>(a.N) * a.H * (a.dv / 16);
  int best = 2;
  double best_t = 0.0;
  const int cand[4] = {1, 2, 4, 8};
  const double step[4] = {0.92, 1.0, 1.29, 2.06};
  for (int i = 0; i < 4; ++i) {
    if (a.dv % (16 * cand[i]) != 0) continue;
    const int64_t wgs = slabs / cand[i];
    const double t = static_cast<double>((wgs + kCUs - 1) / kCUs) * step[i];
    if (i == 0 || t < best_t) {
      best = cand[i];
      best_t = t;
    }
  }
  return best;
}

int chunk_fwd_state_columns(const ChunkArgs &a) {
  return a.in_dtype == 0 ? 32 : 16 * prefill_ns(a);
}

template <typename TIN, typename TOUT>
static hipError_t launch_16(const ChunkArgs &a) {
  // runs of the segment-parallel form (in sequence order: the ordering by
  // length is only a scheduling aid)
  const int ns = prefill_ns(a);
  if (!a.seg.plain()) {
    if (ns == 8) return launch_bf16<128, 8, TIN, TOUT, false, false, true>(a);
    if (ns == 4) return launch_bf16<128, 4, TIN, TOUT, false, false, true>(a);
    if (ns == 1) return launch_bf16<128, 1, TIN, TOUT, false, false, true>(a);
    return a.dk == 128 ? launch_bf16<128, 2, TIN, TOUT, false, false, true>(a)
                       : launch_bf16<64, 2, TIN, TOUT, false, false, true>(a);
  }
  if (a.cu_seqlens && a.N > 1 && a.N <= kLptMax) {
    if (ns == 8) return launch_bf16<128, 8, TIN, TOUT, false, true>(a);
    if (ns == 4) return launch_bf16<128, 4, TIN, TOUT, false, true>(a);
    if (ns == 1) return launch_bf16<128, 1, TIN, TOUT, false, true>(a);
    return a.dk == 128 ? launch_bf16<128, 2, TIN, TOUT, false, true>(a)
                       : launch_bf16<64, 2, TIN, TOUT, false, true>(a);
  }
  if (ns == 8) return launch_bf16<128, 8, TIN, TOUT>(a);
  if (ns == 4) return launch_bf16<128, 4, TIN, TOUT>(a);
  if (ns == 1) return launch_bf16<128, 1, TIN, TOUT>(a);
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

hipError_t launch_chunk_fwd_states(const ChunkArgs &a) {
  const int ns = prefill_ns(a);
  if (a.in_dtype == 2) {
    if (ns == 8) return launch_bf16<128, 8, _Float16, _Float16, true>(a);
    if (ns == 4) return launch_bf16<128, 4, _Float16, _Float16, true>(a);
    if (ns == 1) return launch_bf16<128, 1, _Float16, _Float16, true>(a);
    return a.dk == 128 ? launch_bf16<128, 2, _Float16, _Float16, true>(a)
                       : launch_bf16<64, 2, _Float16, _Float16, true>(a);
  }
  if (ns == 8) return launch_bf16<128, 8, bf16_t, bf16_t, true>(a);
  if (ns == 4) return launch_bf16<128, 4, bf16_t, bf16_t, true>(a);
  if (ns == 1) return launch_bf16<128, 1, bf16_t, bf16_t, true>(a);
  return a.dk == 128 ? launch_bf16<128, 2, bf16_t, bf16_t, true>(a)
                     : launch_bf16<64, 2, bf16_t, bf16_t, true>(a);
}

hipError_t launch_chunk_fwd(const ChunkArgs &a) {
  return a.in_dtype == 0 ? launch_chunk_fwd_f32(a) : launch_chunk_fwd_bf16(a);
}

}  // namespace gdn
