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
// head): each thread keeps DK*DV/256 state values in registers (16-byte
// accesses, 4 adjacent columns), so the state never round-trips through LDS
// between tokens; only the per-column partial dot products are reduced
// across row groups, one barrier per token.
//
// Gates arrive either as log alpha and beta or as raw pre-activations that
// are turned into gates here (RawGate). For serving, the states may live in
// a pool of slots (see DecodeArgs): a sequence reads one slot, and writes
// its final state back there or, for speculative verification, the state
// after each token into a slot of its own.
//
// The fused variant also runs the mixer's front end and output gate (page
// "NLP——技术报告解读-Qwen3.8-Flash-Next", section "GDN 参数化细节"): it takes
// the raw projections, applies the short causal convolution with the three
// previous raw rows kept per slot (conv_state), SiLU, and the L2 norm of q
// and k, and writes o = sigmoid(z) * RMSNorm(y) * (1 + w) instead of y. That
// work is per (sequence, head) and small; it adds the raw rows, z and the
// conv cache (~3% of the bytes at d = 128) to the stream.
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

template <int DK, int DV, typename TIN, typename TOUT, bool FUSED>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a) {
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

template <int DK, int DV, typename TIN, typename TOUT, bool FUSED>
static hipError_t launch(const DecodeArgs &a) {
  const int units = a.N * a.H;
  if (units == 0 || a.n_tok <= 0) return hipSuccess;
  hipLaunchKernelGGL((decode_kernel<DK, DV, TIN, TOUT, FUSED>), dim3(units), dim3(256), 0,
                     a.stream, a);
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
