// Decode steps of the gated delta rule (gfx950).
//
// Each token updates the fixed-size fp32 state of its (sequence, head) in
// place (page "NLP——技术报告解读-Qwen3.8-Flash-Next", section "Gated DeltaNet
// 核心机制"):
//     S~ = alpha S;  e = v - S~^T k;  S = S~ + beta k e^T;  y = S^T q.
// Per column j of S this needs the two dot products s_j.k and s_j.q over the
// key dimension, so
//     e_j = v_j - alpha (s_j.k),    y_j = alpha (s_j.q) + beta (k.q) e_j,
//     s_j <- alpha s_j + beta e_j k.
// A call applies n_tok (1..kDecodeMaxTok) consecutive tokens per (sequence,
// head), e.g. a speculative-decoding verify step. The work is a pure HBM
// stream: the state (64 KiB per (sequence, head) at dk = dv = 128) is read
// once and written once per call, however many tokens it applies; the token
// inputs are ~1% of the bytes. One 256-thread workgroup owns one (sequence,
// head) and keeps the state in registers (16-byte accesses, 4 adjacent
// columns per lane), so it never round-trips through LDS between tokens.
// Two kernels:
//   * decode_token_kernel applies the tokens one by one. A wave holds whole
//     rows (all columns), so every 16-byte load or store instruction of a
//     wave covers whole 512-byte rows; the per-column partial dot products
//     are reduced across row groups with one LDS exchange and barrier per
//     token. It serves single tokens and calls that keep the state after
//     every token.
//   * decode_block_kernel applies up to four tokens as one block in the
//     unrolled form below: one pass of dot products against the state and
//     one update per block instead of per token, with a wave holding whole
//     columns, so the row sums stay inside the wave (no barrier). It serves
//     multi-token calls that keep only the final state.
//
// Gates arrive either as log alpha and beta or as raw pre-activations that
// are turned into gates here (RawGate). For serving, the states may live in
// a pool of slots (see DecodeArgs): a sequence reads one slot, and writes
// its final state back there or, for speculative verification, the state
// after each token into a slot of its own.
//
// The fused variants also run the mixer's front end and output gate (page
// "NLP——技术报告解读-Qwen3.8-Flash-Next", section "GDN 参数化细节"): they
// take the raw projections, apply the short causal convolution with the
// three previous raw rows kept per slot (conv_state), SiLU, and the L2 norm
// of q and k, and write o = sigmoid(z) * RMSNorm(y) * (1 + w) instead of y.
// That work is per (sequence, head) and small; it adds the raw rows, z and
// the conv cache (~3% of the bytes at d = 128) to the stream.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// four consecutive elements of a 16- or 32-bit type as floats, and back
template <typename T>
__device__ __forceinline__ void load4(const T *p, float *o) {
  if constexpr (sizeof(T) == 4) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = v[i];
  } else {
    struct alignas(8) R { T v[4]; } r = *reinterpret_cast<const R *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = io<T>::to_f32(r.v[i]);
  }
}
template <typename T>
__device__ __forceinline__ void store4(T *p, const float *v) {
  struct alignas(4 * sizeof(T)) R { T v[4]; } r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.v[i] = io<T>::from_f32(v[i]);
  *reinterpret_cast<R *>(p) = r;
}

__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// one, two or four consecutive floats of LDS in one access
template <int G>
__device__ __forceinline__ void lds_read(const float *p, float *o) {
  if constexpr (G == 4) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = v[i];
  } else if constexpr (G == 2) {
    const float2 v = *reinterpret_cast<const float2 *>(p);
    o[0] = v.x;
    o[1] = v.y;
  } else {
    o[0] = p[0];
  }
}

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t x) { return __builtin_bit_cast(float, x); }

// Sum over the lanes of a wave that agree in lane bits 0..FROM-1, i.e. over
// bits FROM..5; every lane receives its group's total. Bits below 4 are
// summed by DPP rotations inside each 16-lane row, bit 4 by swapping the odd
// rows of one copy with the even rows of another, bit 5 by swapping the wave
// halves of two copies (gfx950 permlane swaps): no LDS traffic.
template <int FROM>
__device__ __forceinline__ float lane_sum(float x) {
  static_assert(FROM >= 0 && FROM <= 4, "lane bits");
  if constexpr (FROM <= 0)
    x += bitsf(__builtin_amdgcn_update_dpp(0u, fbits(x), 0x121, 0xf, 0xf, false));  // row_ror:1
  if constexpr (FROM <= 1)
    x += bitsf(__builtin_amdgcn_update_dpp(0u, fbits(x), 0x122, 0xf, 0xf, false));  // row_ror:2
  if constexpr (FROM <= 2)
    x += bitsf(__builtin_amdgcn_update_dpp(0u, fbits(x), 0x124, 0xf, 0xf, false));  // row_ror:4
  if constexpr (FROM <= 3)
    x += bitsf(__builtin_amdgcn_update_dpp(0u, fbits(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  const auto r16 = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
  x = bitsf(r16[0]) + bitsf(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
  return bitsf(r32[0]) + bitsf(r32[1]);
}

__device__ __forceinline__ float uniform(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// Four per-lane partial sums v[0..3] (the 4 columns of a lane's column
// group) reduced over the row groups at once: the result holds in 16-lane row
// r (lane bits 4, 5) the total of v[r] for the lane's column group. Swapping
// the wave halves of v[0] and v[2] (and v[1], v[3]) and adding leaves rows
// 0-1 with column 0 (1) and rows 2-3 with column 2 (3), halved over bit 5;
// swapping the odd rows of the first sum with the even rows of the second and
// adding sorts column r into row r, summed over bit 4; the row rotations sum
// over the remaining bits FROM..3 of the row group.
template <int FROM>
__device__ __forceinline__ float sum4_rows(const float *v) {
  const auto a = __builtin_amdgcn_permlane32_swap(fbits(v[0]), fbits(v[2]), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(fbits(v[1]), fbits(v[3]), false, false);
  const float x = bitsf(a[0]) + bitsf(a[1]);
  const float y = bitsf(b[0]) + bitsf(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(y), false, false);
  float r = bitsf(c[0]) + bitsf(c[1]);
  if constexpr (FROM <= 2)
    r += bitsf(__builtin_amdgcn_update_dpp(0u, fbits(r), 0x124, 0xf, 0xf, false));  // row_ror:4
  r += bitsf(__builtin_amdgcn_update_dpp(0u, fbits(r), 0x128, 0xf, 0xf, false));    // row_ror:8
  return r;
}

// The inverse move: o[r] receives, in every row, what row r of x holds.
__device__ __forceinline__ void bcast_rows(float x, float *o) {
  const auto a = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
  // a[0]: rows (0, 0, 2, 2); a[1]: rows (1, 1, 3, 3)
  const auto b = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);
  const auto c = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);
  o[0] = bitsf(b[0]);
  o[2] = bitsf(b[1]);
  o[1] = bitsf(c[0]);
  o[3] = bitsf(c[1]);
}

// a barrier for LDS traffic only: loads into registers stay in flight
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int DK, int DV, typename TIN, typename TOUT, bool FUSED>
__global__ __launch_bounds__(256) void decode_token_kernel(const DecodeArgs a) {
  const TIN *__restrict__ q = static_cast<const TIN *>(a.q);
  const TIN *__restrict__ k = static_cast<const TIN *>(a.k);
  const TIN *__restrict__ v = static_cast<const TIN *>(a.v);
  const float *__restrict__ ga = a.log_alpha;
  const float *__restrict__ gb = a.beta;
  float *__restrict__ S = a.S;
  const int32_t *__restrict__ read_idx = a.read_idx;
  const int32_t *__restrict__ write_idx = a.write_idx;
  const int r_stride = a.r_stride, w_stride = a.w_stride, n_slots = a.n_slots;
  TOUT *__restrict__ y = static_cast<TOUT *>(a.y);
  const int H = a.H, n_tok = a.n_tok;
  constexpr int NT = 256;
  constexpr int CG = DV / 4;   // column groups of 4 adjacent columns
  constexpr int RG = NT / CG;  // row groups
  constexpr int RPT = DK / RG; // rows per thread
  constexpr int RG_PER_WAVE = 64 / CG;
  constexpr int NWAVE = NT / 64;
  static_assert(DK % RG == 0 && RG_PER_WAVE >= 1, "shape");
  static_assert(!FUSED || DK == DV, "the fused front end needs dk == dv");

  __shared__ float sq[kDecodeMaxTok][DK];
  __shared__ float sk[kDecodeMaxTok][DK];
  __shared__ float sv[kDecodeMaxTok][DV];
  __shared__ float s_alpha[kDecodeMaxTok], s_beta[kDecodeMaxTok];
  __shared__ float red[2][NWAVE][CG][9];
  __shared__ float sz[FUSED ? kDecodeMaxTok : 1][DV];

  const int unit = blockIdx.x;  // n * H + h
  const int n = unit / H;
  const int h = unit - n * H;
  const int tid = threadIdx.x;
  const int cg = tid % CG;
  const int rg = tid / CG;
  const int wave = tid / 64;

  int slot = n;
  if (read_idx) {
    slot = read_idx[static_cast<int64_t>(n) * r_stride];
    if (slot < 0 || slot >= n_slots) {
      // padding entry: no state to update; y (or o) = 0
      for (int idx = tid; idx < n_tok * DV; idx += NT) {
        const size_t row = static_cast<size_t>(n) * n_tok + idx / DV;
        y[(row * H + h) * DV + idx % DV] = io<TOUT>::from_f32(0.0f);
      }
      return;
    }
  }
  // State accesses go through a buffer resource per (slot, head): one lane
  // offset register and a scalar offset per row step, instead of a 64-bit
  // address per access. aux = 2 marks them non-temporal (streamed once).
  auto state_rsrc = [&](int64_t sl) {
    return __builtin_amdgcn_make_buffer_rsrc(S + (static_cast<size_t>(sl) * H + h) * DK * DV, 0,
                                             DK * DV * 4, 0x00020000);
  };
  const int s_lane = (rg * DV + 4 * cg) * 4;
  constexpr int kRowStep = RG * DV * 4;
  const auto Sr = state_rsrc(slot);

  // Token inputs go to LDS, one 16-byte load per thread and tensor; with
  // the front end fused these are the raw rows (and z). Nothing here
  // branches (a branch would make the compiler wait inside it): lanes past
  // the last piece are clamped to it and store the same values again.
  constexpr int VEC = io<TIN>::kVec;
  static_assert(kDecodeMaxTok * DK / VEC <= NT && kDecodeMaxTok * DV / VEC <= NT, "lanes");
  const size_t row0 = static_cast<size_t>(n) * n_tok;
  const int pk = min(tid, n_tok * (DK / VEC) - 1);  // piece of q / k
  const int pv = min(tid, n_tok * (DV / VEC) - 1);  // piece of v
  const int jk = pk / (DK / VEC), ck = (pk % (DK / VEC)) * VEC;
  const int jv = pv / (DV / VEC), cv = (pv % (DV / VEC)) * VEC;
  float qf[VEC], kf[VEC], vf[VEC], zf[VEC];
  f32x4 s[RPT];
  auto load_state = [&]() {
#pragma unroll
    for (int m = 0; m < RPT; ++m)
      s[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(Sr, s_lane,
                                                                             m * kRowStep, 2));
  };
  // Without the front end the state loads go first: they are the whole
  // cost of the kernel. With it, the small loads the front end needs go
  // first, so that waiting for them leaves the state loads in flight.
  if constexpr (!FUSED) load_state();
  io<TIN>::load16(q + ((row0 + jk) * H + h) * DK + ck, qf);
  io<TIN>::load16(k + ((row0 + jk) * H + h) * DK + ck, kf);
  io<TIN>::load16(v + ((row0 + jv) * H + h) * DV + cv, vf);
  if constexpr (FUSED)
    io<TIN>::load16(static_cast<const TIN *>(a.z) + ((row0 + jv) * H + h) * DV + cv, zf);
  const int gj = min(tid, n_tok - 1);
  const size_t gi = (row0 + gj) * H + h;
  float la = ga[gi];
  float bt = gb[gi];
  const RawGate gate = RawGate::load(a.A, a.b_alpha, h);

  // front-end lanes: lane f < 3 * FG owns 4 channels of one stream
  // (q, k, v); lanes past them repeat the last one
  constexpr int FG = DK / 4;
  const int fj = min(tid, 3 * FG - 1);
  const int fs = fj / FG;
  const int fc = (fj % FG) * 4;
  float fw[4][4], hist[3][4], nw[4];
  TIN *cstate = nullptr;
  if constexpr (FUSED) {
    const float *wp = a.conv_w + ((static_cast<size_t>(fs) * H + h) * DK + fc) * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 w4 = *reinterpret_cast<const f32x4 *>(wp + 4 * c);
#pragma unroll
      for (int t = 0; t < 4; ++t) fw[c][t] = w4[t];
    }
    cstate = static_cast<TIN *>(a.conv_state);
    const TIN *hp = cstate + ((static_cast<size_t>(slot) * H + h) * 3 + fs) * 3 * DK + fc;
#pragma unroll
    for (int r = 0; r < 3; ++r) load4(hp + r * DK, hist[r]);
#pragma unroll
    for (int c = 0; c < 4; ++c) nw[c] = 1.0f + (a.norm_w ? a.norm_w[4 * cg + c] : 0.0f);
    load_state();
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    sq[jk][ck + e] = qf[e];
    sk[jk][ck + e] = kf[e];
    sv[jv][cv + e] = vf[e];
    if constexpr (FUSED) sz[jv][cv + e] = zf[e];
  }
  if (gate.raw()) {
    la = gate.log_alpha(la);
    bt = RawGate::beta(bt);
  }
  s_alpha[gj] = __expf(la);
  s_beta[gj] = bt;
  __syncthreads();

  if constexpr (FUSED) {
    // Front end, token by token, in place in sq / sk / sv: each lane owns
    // its 4 channels in every row, so nobody else reads or writes them.
    // hist keeps the three previous raw rows, oldest first.
    if (wave * 64 < 3 * FG) {
      float *const row_base = fs == 0 ? &sq[0][0] : (fs == 1 ? &sk[0][0] : &sv[0][0]);
      for (int j = 0; j < n_tok; ++j) {
        float *const rp = row_base + j * DK + fc;
        float x[4], u[4], ss = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[c] = rp[c];
          const float acc = fw[c][0] * hist[0][c] + fw[c][1] * hist[1][c] +
                            fw[c][2] * hist[2][c] + fw[c][3] * x[c];
          u[c] = acc * sigmoid_fast(acc);
          ss = fmaf(u[c], u[c], ss);
        }
        // sum of squares over the stream's FG lanes (aligned lane groups)
#pragma unroll
        for (int off = 1; off < FG; off <<= 1) ss += __shfl_xor(ss, off, 64);
        const float scale = fs < 2 ? rsqrtf(ss + a.l2_eps) : 1.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          rp[c] = u[c] * scale;
          hist[0][c] = hist[1][c];
          hist[1][c] = hist[2][c];
          hist[2][c] = x[c];
        }
        // the convolution history after token j goes wherever the state
        // after token j goes
        int dst = -1;
        if (write_idx) {
          const int ws = write_idx[static_cast<int64_t>(n) * w_stride + j];
          if (ws >= 0 && ws < n_slots) dst = ws;
        } else if (j == n_tok - 1) {
          dst = slot;
        }
        if (dst >= 0 && tid < 3 * FG) {
          TIN *hp = cstate + ((static_cast<size_t>(dst) * H + h) * 3 + fs) * 3 * DK + fc;
#pragma unroll
          for (int r = 0; r < 3; ++r) store4(hp + r * DK, hist[r]);
        }
      }
    }
    __syncthreads();
  }

  auto token = [&](const int j) __attribute__((always_inline)) {
    // partial dot products over this thread's rows: s_j.k, s_j.q (4 columns)
    // and k.q (the same for every column group)
    float p[9];
#pragma unroll
    for (int c = 0; c < 9; ++c) p[c] = 0.0f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int i = rg + RG * m;
      const float ki = sk[j][i];
      const float qi = sq[j][i];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        p[c] = fmaf(s[m][c], ki, p[c]);
        p[4 + c] = fmaf(s[m][c], qi, p[4 + c]);
      }
      p[8] = fmaf(ki, qi, p[8]);
    }
    // reduce over the row groups inside the wave (lanes that differ by CG)
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
      for (int c = 0; c < 9; ++c) p[c] += __shfl_xor(p[c], off, 64);
    }
    // red is double-buffered by token parity: buffer j & 1 was last read
    // before the previous token's barrier, which every thread has passed
    if ((tid % 64) < CG) {
#pragma unroll
      for (int c = 0; c < 9; ++c) red[j & 1][wave][cg][c] = p[c];
    }
    __syncthreads();
    float tot[9];
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) acc += red[j & 1][w][cg][c];
      tot[c] = acc;
    }

    const float alpha = s_alpha[j];
    const float b = s_beta[j];
    float e[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) e[c] = sv[j][4 * cg + c] - alpha * tot[c];
    if (rg == 0) {
      // the 4 adjacent outputs of this column group in one store
      float yv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) yv[c] = alpha * tot[4 + c] + b * tot[8] * e[c];
      if constexpr (FUSED) {
        // output gate: RMS over the row's DV values, held by the CG lanes
        // with rg == 0 (an aligned lane group)
        float ss = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) ss = fmaf(yv[c], yv[c], ss);
#pragma unroll
        for (int off = 1; off < CG; off <<= 1) ss += __shfl_xor(ss, off, 64);
        const float inv = rsqrtf(ss * (1.0f / DV) + a.rms_eps);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          yv[c] = yv[c] * inv * nw[c] * sigmoid_fast(sz[j][4 * cg + c]);
      }
      store4(y + ((row0 + j) * H + h) * DV + 4 * cg, yv);
    }
    float be[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) be[c] = b * e[c];
    // where the state after this token goes, if anywhere; each row is
    // stored as soon as it is updated, so the stores drain while the rest
    // of the update still runs
    bool store = !write_idx && j == n_tok - 1;
    int dst = slot;
    if (write_idx) {
      dst = write_idx[static_cast<int64_t>(n) * w_stride + j];
      store = dst >= 0 && dst < n_slots;
    }
    const auto Sw = state_rsrc(store ? dst : slot);
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const float ki = sk[j][rg + RG * m];
#pragma unroll
      for (int c = 0; c < 4; ++c) s[m][c] = fmaf(alpha, s[m][c], be[c] * ki);
      if (store)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[m]), Sw, s_lane,
                                               m * kRowStep, 2);
    }
  };
  // token 0 is peeled off the loop: entering the loop with the freshly
  // loaded state made the compiler copy all of it into separate
  // loop-carried registers, which costs occupancy
  token(0);
  for (int j = 1; j < n_tok; ++j) token(j);
}

// Blocks of G = 4 tokens (the last one padded with zero tokens). Within a block
// that starts from state S, with cum_t the running sum of log alpha over the
// block (Gam_t = exp(cum_t)) and D_ti = exp(cum_t - cum_i), unrolling the
// recurrence gives, per column j:
//     e_t = v_tj - Gam_t (s_j.k_t) - sum_{i<t} D_ti beta_i (k_i.k_t) e_i
//     y_t = Gam_t (s_j.q_t) + sum_{i<=t} D_ti beta_i (k_i.q_t) e_i
//     s_j <- Gam_{G-1} s_j + sum_i D_{G-1,i} beta_i e_i k_i,
// so the state is touched by one pass of dot products (all 2G of them) and
// one update per block, and only 2G sums per column cross lanes.
template <int DK, int DV, typename TIN, typename TOUT, bool FUSED>
__global__ __launch_bounds__(256, FUSED ? 3 : 4) void decode_block_kernel(const DecodeArgs a) {
  constexpr int G = 4;  // tokens per block
  const TIN *__restrict__ q = static_cast<const TIN *>(a.q);
  const TIN *__restrict__ k = static_cast<const TIN *>(a.k);
  const TIN *__restrict__ v = static_cast<const TIN *>(a.v);
  const float *__restrict__ ga = a.log_alpha;
  const float *__restrict__ gb = a.beta;
  float *__restrict__ S = a.S;
  const int32_t *__restrict__ read_idx = a.read_idx;
  const int32_t *__restrict__ write_idx = a.write_idx;
  const int r_stride = a.r_stride, w_stride = a.w_stride, n_slots = a.n_slots;
  TOUT *__restrict__ y = static_cast<TOUT *>(a.y);
  const int H = a.H, n_tok = a.n_tok;
  constexpr int NT = 256;
  constexpr int NWAVE = NT / 64;
  constexpr int CPW = DV / NWAVE;    // columns per wave
  constexpr int CGW = CPW / 4;       // column groups (4 adjacent columns) per wave
  constexpr int RGW = 64 / CGW;      // row groups per wave
  constexpr int RPT = DK / RGW;      // rows per lane
  constexpr int TP = kDecodeMaxTok;  // token slots in LDS
  static_assert((CGW == 4 || CGW == 8) && DK % RGW == 0, "shape");
  static_assert(TP % G == 0, "block");
  static_assert(!FUSED || DK == DV, "the fused front end needs dk == dv");
  constexpr int CGB = CGW == 8 ? 3 : 2;  // lane bits of the column group
  // Gram entries of a block: k_i.k_t for i < t, then k_i.q_t for i <= t
  constexpr int NKK = G * (G - 1) / 2;
  constexpr int NKQ = G * (G + 1) / 2;
  static_assert(DK % 64 == 0, "Gram rows");

  // q and k token-minor, so that one 16-byte read gives a row of 4 tokens
  __shared__ __align__(16) float sqT[DK][TP];
  __shared__ __align__(16) float skT[DK][TP];
  __shared__ __align__(16) float sv[TP][DV];
  __shared__ float s_la[TP], s_beta[TP];
  __shared__ int s_dst[TP];  // slot receiving the state after token t, or -1
  __shared__ __align__(16) float sz[FUSED ? TP : 1][DV];
  __shared__ float s_ss[FUSED ? TP : 1][NWAVE];

  const int unit = blockIdx.x;  // n * H + h
  const int n = unit / H;
  const int h = unit - n * H;
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int cg = lane % CGW;
  const int rg = lane / CGW;
  const int col0 = wave * CPW + 4 * cg;
  const int cr = (lane >> 4) & 3;            // a column of the group, after the row sums
  const bool col_lead = (lane & 15) < CGW;   // the first lane holding that column

  int slot = n;
  if (read_idx) {
    slot = read_idx[static_cast<int64_t>(n) * r_stride];
    if (slot < 0 || slot >= n_slots) {
      // padding entry: no state to update; y (or o) = 0
      for (int idx = tid; idx < n_tok * DV; idx += NT) {
        const size_t row = static_cast<size_t>(n) * n_tok + idx / DV;
        y[(row * H + h) * DV + idx % DV] = io<TOUT>::from_f32(0.0f);
      }
      return;
    }
  }
  // Token slots past the call's tokens, up to a whole block, hold zeros:
  // k = q = v = 0 and beta = 0 leave the state alone, log alpha = 0 keeps
  // the decay. Written before any load is issued.
  const int n_pad = (n_tok + G - 1) / G * G;
  {
    constexpr int PER = 2 * DK + DV;
    for (int idx = tid; idx < (n_pad - n_tok) * PER; idx += NT) {
      const int t = n_tok + idx / PER, r = idx % PER;
      if (r < DK) sqT[r][t] = 0.0f;
      else if (r < 2 * DK) skT[r - DK][t] = 0.0f;
      else sv[t][r - 2 * DK] = 0.0f;
    }
  }
  // State accesses go through a buffer resource per (slot, head): one lane
  // offset register and a scalar offset per row step, instead of a 64-bit
  // address per access. aux = 2 marks them non-temporal (streamed once).
  // Lane (cg, rg) of wave w holds rows rg + RGW m, columns col0..col0+3.
  auto state_rsrc = [&](int64_t sl) {
    return __builtin_amdgcn_make_buffer_rsrc(S + (static_cast<size_t>(sl) * H + h) * DK * DV, 0,
                                             DK * DV * 4, 0x00020000);
  };
  const int s_lane = (rg * DV + col0) * 4;
  constexpr int kRowStep = RGW * DV * 4;
  const auto Sr = state_rsrc(slot);

  // Token inputs go to LDS, one 16-byte load per thread and tensor; with
  // the front end fused these are the raw rows (and z). Nothing here
  // branches (a branch would make the compiler wait inside it): lanes past
  // the last piece are clamped to it and store the same values again. These
  // small loads go first, the state loads after them, so that the inputs
  // can be used (the Gram entries below) while the state is in flight.
  constexpr int VEC = io<TIN>::kVec;
  static_assert(kDecodeMaxTok * DK / VEC <= NT && kDecodeMaxTok * DV / VEC <= NT, "lanes");
  const size_t row0 = static_cast<size_t>(n) * n_tok;
  const int pk = min(tid, n_tok * (DK / VEC) - 1);  // piece of q / k
  const int pv = min(tid, n_tok * (DV / VEC) - 1);  // piece of v
  const int jk = pk / (DK / VEC), ck = (pk % (DK / VEC)) * VEC;
  const int jv = pv / (DV / VEC), cv = (pv % (DV / VEC)) * VEC;
  float qf[VEC], kf[VEC], vf[VEC], zf[VEC];
  f32x4 s[RPT];
  io<TIN>::load16(q + ((row0 + jk) * H + h) * DK + ck, qf);
  io<TIN>::load16(k + ((row0 + jk) * H + h) * DK + ck, kf);
  io<TIN>::load16(v + ((row0 + jv) * H + h) * DV + cv, vf);
  if constexpr (FUSED)
    io<TIN>::load16(static_cast<const TIN *>(a.z) + ((row0 + jv) * H + h) * DV + cv, zf);
  const int gj = min(tid, n_tok - 1);
  const size_t gi = (row0 + gj) * H + h;
  float la = ga[gi];
  float bt = gb[gi];
  const RawGate gate = RawGate::load(a.A, a.b_alpha, h);
  // the slot table's write entries, read with the small loads (without a
  // table the gates are read in their place, and the value is not used)
  const int32_t *wtab = write_idx ? write_idx + static_cast<int64_t>(n) * w_stride
                                  : reinterpret_cast<const int32_t *>(ga);
  const int wraw = wtab[gj];

  // front-end lanes: lane f < 3 * FG owns 4 channels of one stream
  // (q, k, v); lanes past them repeat the last one
  constexpr int FG = DK / 4;
  const int fj = min(tid, 3 * FG - 1);
  const int fs = fj / FG;
  const int fc = (fj % FG) * 4;
  float fw[4][4], hist[3][4], nw = 0.0f;
  TIN *cstate = nullptr;
  if constexpr (FUSED) {
    const float *wp = a.conv_w + ((static_cast<size_t>(fs) * H + h) * DK + fc) * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 w4 = *reinterpret_cast<const f32x4 *>(wp + 4 * c);
#pragma unroll
      for (int t = 0; t < 4; ++t) fw[c][t] = w4[t];
    }
    cstate = static_cast<TIN *>(a.conv_state);
    const TIN *hp = cstate + ((static_cast<size_t>(slot) * H + h) * 3 + fs) * 3 * DK + fc;
#pragma unroll
    for (int r = 0; r < 3; ++r) load4(hp + r * DK, hist[r]);
    nw = 1.0f + (a.norm_w ? a.norm_w[col0 + cr] : 0.0f);
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m)
    s[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(Sr, s_lane,
                                                                           m * kRowStep, 2));
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    sqT[ck + e][jk] = qf[e];
    skT[ck + e][jk] = kf[e];
    sv[jv][cv + e] = vf[e];
    if constexpr (FUSED) sz[jv][cv + e] = zf[e];
  }
  if (gate.raw()) {
    la = gate.log_alpha(la);
    bt = RawGate::beta(bt);
  }
  if (tid < TP) {
    s_la[tid] = tid < n_tok ? la : 0.0f;
    s_beta[tid] = tid < n_tok ? bt : 0.0f;
    s_dst[tid] = write_idx ? (tid < n_tok && wraw >= 0 && wraw < n_slots ? wraw : -1)
                           : (tid == n_tok - 1 ? slot : -1);
  }
  lds_barrier();

  if constexpr (FUSED) {
    // Front end, token by token, in place in LDS: each lane owns its 4
    // channels in every token, so nobody else reads or writes them. hist
    // keeps the three previous raw rows, oldest first.
    if (wave * 64 < 3 * FG) {
      float *const fbase = fs == 0 ? &sqT[fc][0] : (fs == 1 ? &skT[fc][0] : &sv[0][fc]);
      const int sj = fs == 2 ? DV : 1;  // token stride
      const int sc = fs == 2 ? 1 : TP;  // channel stride
      for (int j = 0; j < n_tok; ++j) {
        float *const rp = fbase + j * sj;
        float x[4], u[4], ss = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[c] = rp[c * sc];
          const float acc = fw[c][0] * hist[0][c] + fw[c][1] * hist[1][c] +
                            fw[c][2] * hist[2][c] + fw[c][3] * x[c];
          u[c] = acc * sigmoid_fast(acc);
          ss = fmaf(u[c], u[c], ss);
        }
        // sum of squares over the stream's FG lanes (aligned lane groups)
#pragma unroll
        for (int off = 1; off < FG; off <<= 1) ss += __shfl_xor(ss, off, 64);
        const float scale = fs < 2 ? rsqrtf(ss + a.l2_eps) : 1.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          rp[c * sc] = u[c] * scale;
          hist[0][c] = hist[1][c];
          hist[1][c] = hist[2][c];
          hist[2][c] = x[c];
        }
        // the convolution history after token j goes wherever the state
        // after token j goes
        const int dst = s_dst[j];
        if (dst >= 0 && tid < 3 * FG) {
          TIN *hp = cstate + ((static_cast<size_t>(dst) * H + h) * 3 + fs) * 3 * DK + fc;
#pragma unroll
          for (int r = 0; r < 3; ++r) store4(hp + r * DK, hist[r]);
        }
      }
    }
    lds_barrier();
  }

  const int n_blk = n_pad / G;
  static_assert(TP / G <= 2, "at most two blocks per call");
  // Per block: cum_t, the running sum of log alpha over the block, and
  // Gam_t = exp(cum_t); the Gram entries, summed by every wave on its own
  // (lane l takes rows l, l + 64, ...), and their coefficients
  // D_ti beta_i (k_i . x_t). All uniform (scalar registers) and independent
  // of the state, so they are formed while the state loads are in flight:
  // without the front end both blocks' sets up front, with it (which holds
  // more registers) each block's own just before it.
  struct Coef {
    float cum[G], Gam[G], ckk[NKK > 0 ? NKK : 1], ckq[NKQ];
  };
  auto coef_of = [&](const int t0) __attribute__((always_inline)) {
    Coef cf;
    {
      float acc = 0.0f;
#pragma unroll
      for (int t = 0; t < G; ++t) {
        acc += s_la[t0 + t];
        cf.cum[t] = uniform(acc);
        cf.Gam[t] = uniform(__expf(acc));
      }
    }
    float gk[NKK > 0 ? NKK : 1], gq[NKQ];
#pragma unroll
    for (int p = 0; p < NKK; ++p) gk[p] = 0.0f;
#pragma unroll
    for (int p = 0; p < NKQ; ++p) gq[p] = 0.0f;
#pragma unroll
    for (int m = 0; m < DK / 64; ++m) {
      float kr[G], qr[G];
      lds_read<G>(&skT[lane + 64 * m][t0], kr);
      lds_read<G>(&sqT[lane + 64 * m][t0], qr);
#pragma unroll
      for (int t = 0; t < G; ++t)
#pragma unroll
        for (int i = 0; i <= t; ++i) {
          if (i < t) gk[t * (t - 1) / 2 + i] = fmaf(kr[i], kr[t], gk[t * (t - 1) / 2 + i]);
          gq[t * (t + 1) / 2 + i] = fmaf(kr[i], qr[t], gq[t * (t + 1) / 2 + i]);
        }
    }
    float bet[G];
#pragma unroll
    for (int i = 0; i < G; ++i) bet[i] = s_beta[t0 + i];
#pragma unroll
    for (int t = 0; t < G; ++t)
#pragma unroll
      for (int i = 0; i <= t; ++i) {
        // D_ti beta_i = exp(cum_t - cum_i) beta_i
        const float db = i == t ? bet[i] : __expf(cf.cum[t] - cf.cum[i]) * bet[i];
        if (i < t) cf.ckk[t * (t - 1) / 2 + i] = uniform(db * lane_sum<0>(gk[t * (t - 1) / 2 + i]));
        cf.ckq[t * (t + 1) / 2 + i] = uniform(db * lane_sum<0>(gq[t * (t + 1) / 2 + i]));
      }
    return cf;
  };

  auto block = [&](const int b, const Coef &cf) __attribute__((always_inline)) {
    const int t0 = b * G;
    const float *cum = cf.cum, *Gam = cf.Gam, *ckk = cf.ckk, *ckq = cf.ckq;

    // s_j . k_t and s_j . q_t over this lane's rows, summed over row groups
    float dk_[G][4], dq_[G][4];
#pragma unroll
    for (int t = 0; t < G; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) dk_[t][c] = dq_[t][c] = 0.0f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      float kr[G], qr[G];
      lds_read<G>(&skT[rg + RGW * m][t0], kr);
      lds_read<G>(&sqT[rg + RGW * m][t0], qr);
#pragma unroll
      for (int t = 0; t < G; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          dk_[t][c] = fmaf(s[m][c], kr[t], dk_[t][c]);
          dq_[t][c] = fmaf(s[m][c], qr[t], dq_[t][c]);
        }
    }
    // From here on a lane works on one column, col0 + cr with cr its row
    // of 16 lanes: the lanes of that row whose bits CGB..3 are zero hold a
    // column group's values, the others the same values again.
    float e[G], yv[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
      const float sk = sum4_rows<CGB>(dk_[t]);
      const float sq = sum4_rows<CGB>(dq_[t]);
      float r = sv[t0 + t][col0 + cr] - Gam[t] * sk;
#pragma unroll
      for (int i = 0; i < t; ++i) r = fmaf(-ckk[t * (t - 1) / 2 + i], e[i], r);
      e[t] = r;
      float o = Gam[t] * sq;
#pragma unroll
      for (int i = 0; i <= t; ++i) o = fmaf(ckq[t * (t + 1) / 2 + i], e[i], o);
      yv[t] = o;
    }
    if constexpr (FUSED) {
      // output gate: the RMS over a row's DV values needs every wave's
      // columns; one LDS exchange per block
#pragma unroll
      for (int t = 0; t < G; ++t) {
        const float ss = lane_sum<0>(col_lead ? yv[t] * yv[t] : 0.0f);
        if (lane == 0) s_ss[t0 + t][wave] = ss;
      }
      lds_barrier();
#pragma unroll
      for (int t = 0; t < G; ++t) {
        float ss = 0.0f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) ss += s_ss[t0 + t][w];
        const float inv = rsqrtf(ss * (1.0f / DV) + a.rms_eps);
        yv[t] = yv[t] * inv * nw * sigmoid_fast(sz[t0 + t][col0 + cr]);
      }
    }
#pragma unroll
    for (int t = 0; t < G; ++t)
      if (col_lead && t0 + t < n_tok)
        y[((row0 + t0 + t) * H + h) * DV + col0 + cr] = io<TOUT>::from_f32(yv[t]);

    // where the state after token t goes (s_dst: its slot from the table,
    // or without a table the starting slot after the call's last token; -1
    // for nowhere)
    auto dst_of = [&](int t) { return s_dst[t]; };
    // The state after the block's last real token is the updated state
    // (padding tokens change nothing). The states after earlier tokens of
    // the block are needed only with a table that names slots for them; each
    // is formed from the block's start state in a pass of its own,
    //     S_t = Gam_t S + sum_{i<=t} D_ti beta_i e_i k_i^T.
    const int t_end = min(t0 + G, n_tok) - 1;  // the block's last real token
    if (write_idx) {
#pragma unroll
      for (int t = 0; t < G - 1; ++t) {
        if (t0 + t >= t_end) break;
        const int dt = dst_of(t0 + t);
        if (dt < 0) continue;
        float ut[G][4];
#pragma unroll
        for (int i = 0; i <= t; ++i) {
          const float wi = (i == t ? 1.0f : __expf(cum[t] - cum[i])) * s_beta[t0 + i];
          bcast_rows(wi * e[i], ut[i]);
        }
        const auto St = state_rsrc(dt);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
          float kr[G];
          lds_read<G>(&skT[rg + RGW * m][t0], kr);
          f32x4 x;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            float acc = Gam[t] * s[m][c];
#pragma unroll
            for (int i = 0; i <= t; ++i) acc = fmaf(kr[i], ut[i][c], acc);
            x[c] = acc;
          }
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), St, s_lane,
                                                 m * kRowStep, 2);
        }
      }
    }

    // state update; each row is stored as soon as it is updated, so the
    // stores drain while the rest of the update still runs
    float u[G][4];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float wi = (i == G - 1 ? 1.0f : __expf(cum[G - 1] - cum[i])) * s_beta[t0 + i];
      bcast_rows(wi * e[i], u[i]);
    }
    const int dend = dst_of(t_end);
    const bool store = dend >= 0;
    const auto Sw = state_rsrc(store ? dend : slot);
    const float gl = Gam[G - 1];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      float kr[G];
      lds_read<G>(&skT[rg + RGW * m][t0], kr);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x = gl * s[m][c];
#pragma unroll
        for (int i = 0; i < G; ++i) x = fmaf(kr[i], u[i][c], x);
        s[m][c] = x;
      }
      if (store)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[m]), Sw, s_lane,
                                               m * kRowStep, 2);
    }
  };
  // the scheduler must not sink the coefficient work below the state's dot
  // products, where it would wait for the state and hold registers
  if constexpr (FUSED) {
    {
      const Coef cf = coef_of(0);
      __builtin_amdgcn_sched_barrier(0);
      block(0, cf);
    }
    if (n_blk > 1) {
      const Coef cf = coef_of(G);
      __builtin_amdgcn_sched_barrier(0);
      block(1, cf);
    }
  } else {
    const Coef cf0 = coef_of(0);
    Coef cf1 = cf0;
    if (n_blk > 1) cf1 = coef_of(G);
    __builtin_amdgcn_sched_barrier(0);
    block(0, cf0);
    if (n_blk > 1) block(1, cf1);
  }
}

constexpr unsigned kFusedLdsPad = 30000;  // bytes of dynamic LDS, see launch()

template <int DK, int DV, typename TIN, typename TOUT, bool FUSED>
static hipError_t launch(const DecodeArgs &a) {
  const int units = a.N * a.H;
  if (units == 0 || a.n_tok <= 0) return hipSuccess;
  // one token: token by token; more: in blocks
  if (a.n_tok == 1)
    hipLaunchKernelGGL((decode_token_kernel<DK, DV, TIN, TOUT, FUSED>), dim3(units), dim3(256), 0,
                       a.stream, a);
  else
    // The fused d = 128 variant runs faster with three workgroups per CU than
    // with the four its registers allow (195 against 205 us for 256 x 32
    // states and 4 tokens; the plain variant is fastest at four): unused
    // dynamic LDS, 45 KiB per workgroup in all, keeps the fourth off.
    hipLaunchKernelGGL((decode_block_kernel<DK, DV, TIN, TOUT, FUSED>), dim3(units), dim3(256),
                       FUSED && DK == 128 ? kFusedLdsPad : 0u, a.stream, a);
  return hipGetLastError();
}

template <typename TIN, typename TOUT, bool FUSED>
static hipError_t launch_d(const DecodeArgs &a) {
  if constexpr (FUSED) {
    return a.dk == 128 ? launch<128, 128, TIN, TOUT, true>(a) : launch<64, 64, TIN, TOUT, true>(a);
  } else {
    if (a.dk == 128 && a.dv == 128) return launch<128, 128, TIN, TOUT, false>(a);
    if (a.dk == 128 && a.dv == 64) return launch<128, 64, TIN, TOUT, false>(a);
    if (a.dk == 64 && a.dv == 128) return launch<64, 128, TIN, TOUT, false>(a);
    return launch<64, 64, TIN, TOUT, false>(a);
  }
}

template <typename TIN, bool FUSED>
static hipError_t launch_d_out(const DecodeArgs &a) {
  switch (a.out_dtype) {
    case 1: return launch_d<TIN, bf16_t, FUSED>(a);
    case 2: return launch_d<TIN, _Float16, FUSED>(a);
    default: return launch_d<TIN, float, FUSED>(a);
  }
}

template <bool FUSED>
static hipError_t launch_in(const DecodeArgs &a) {
  if (a.n_tok < 1 || a.n_tok > kDecodeMaxTok) return hipErrorInvalidValue;
  switch (a.in_dtype) {
    case 1: return launch_d_out<bf16_t, FUSED>(a);
    case 2: return launch_d_out<_Float16, FUSED>(a);
    default: return launch_d_out<float, FUSED>(a);
  }
}

hipError_t launch_decode_step(const DecodeArgs &a) { return launch_in<false>(a); }

hipError_t launch_decode_fused(const DecodeArgs &a) {
  if (a.dk != a.dv) return hipErrorInvalidValue;
  return launch_in<true>(a);
}

}  // namespace gdn
