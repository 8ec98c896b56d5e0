// Single-token decode step of the gated delta rule (gfx950).
//
// One token per (sequence, head) updates the fixed-size fp32 state in place
// (page "NLP——技术报告解读-Qwen3.8-Flash-Next", section "Gated DeltaNet 核心机制"):
//     S~ = alpha S;  e = v - S~^T k;  S = S~ + beta k e^T;  y = S^T q.
// Per column j of S this needs the two dot products s_j.k and s_j.q over the
// key dimension, so
//     e_j = v_j - alpha (s_j.k),    y_j = alpha (s_j.q) + beta (k.q) e_j,
//     s_j <- alpha s_j + beta e_j k.
// The step is a pure HBM stream: the state (64 KiB per (sequence, head) at
// dk = dv = 128) is read once and written once; everything else is ~1% of
// the bytes. One 256-thread workgroup owns one (sequence, head): each thread
// keeps DK*DV/256 state values in registers (16-byte accesses, 4 adjacent
// columns), so the read-modify-write never round-trips through LDS; only the
// per-column partial dot products are reduced across row groups.
//
// Gates arrive either as log alpha and beta or as raw pre-activations that
// are turned into gates here (RawGate). For serving, the states may live in
// a pool of slots: sequence n then updates slot state_idx[n], and a sequence
// whose slot is out of range leaves the pool untouched and gets y = 0.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int DK, int DV, typename TIN, typename TOUT>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const TIN *__restrict__ q, const TIN *__restrict__ k, const TIN *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    const float *__restrict__ gA, const float *__restrict__ gbias, float *__restrict__ S,
    const int32_t *__restrict__ state_idx, int n_slots, TOUT *__restrict__ y, int H) {
  constexpr int NT = 256;
  constexpr int CG = DV / 4;   // column groups of 4 adjacent columns
  constexpr int RG = NT / CG;  // row groups
  constexpr int RPT = DK / RG; // rows per thread
  constexpr int RG_PER_WAVE = 64 / CG;
  constexpr int NWAVE = NT / 64;
  static_assert(DK % RG == 0 && RG_PER_WAVE >= 1, "shape");

  __shared__ float sq[DK];
  __shared__ float sk[DK];
  __shared__ float red[NWAVE][CG][9];

  const int unit = blockIdx.x;  // n * H + h
  const int tid = threadIdx.x;
  const int cg = tid % CG;
  const int rg = tid / CG;
  const int wave = tid / 64;

  int64_t slot_unit = unit;
  if (state_idx) {
    const int n = unit / H;
    const int slot = state_idx[n];
    if (slot < 0 || slot >= n_slots) {
      // padding entry: no state to update; y = 0
      const size_t y_off = static_cast<size_t>(unit) * DV;
      for (int j = tid; j < DV; j += NT) y[y_off + j] = io<TOUT>::from_f32(0.0f);
      return;
    }
    slot_unit = static_cast<int64_t>(slot) * H + (unit - n * H);
  }
  float *Su = S + static_cast<size_t>(slot_unit) * DK * DV;

  // issue every state load first: they are the whole cost of the kernel
  f32x4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + RG * m;
    s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Su + i * DV + 4 * cg));
  }

  const size_t qk_off = static_cast<size_t>(unit) * DK;
  for (int i = tid; i < DK; i += NT) {
    sq[i] = io<TIN>::to_f32(q[qk_off + i]);
    sk[i] = io<TIN>::to_f32(k[qk_off + i]);
  }
  const RawGate rg_h = RawGate::load(gA, gbias, unit % H);
  float la = log_alpha[unit];
  float b = beta[unit];
  if (rg_h.raw()) {
    la = rg_h.log_alpha(la);
    b = RawGate::beta(b);
  }
  const float alpha = __expf(la);
  __syncthreads();

  // partial dot products over this thread's rows: s_j.k, s_j.q (4 columns)
  // and k.q (the same for every column group)
  float p[9];
#pragma unroll
  for (int c = 0; c < 9; ++c) p[c] = 0.0f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + RG * m;
    const float ki = sk[i];
    const float qi = sq[i];
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
  if ((tid % 64) < CG) {
#pragma unroll
    for (int c = 0; c < 9; ++c) red[wave][cg][c] = p[c];
  }
  __syncthreads();
  float tot[9];
#pragma unroll
  for (int c = 0; c < 9; ++c) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) acc += red[w][cg][c];
    tot[c] = acc;
  }

  const size_t v_off = static_cast<size_t>(unit) * DV + 4 * cg;
  float e[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float vj = io<TIN>::to_f32(v[v_off + c]);
    e[c] = vj - alpha * tot[c];
  }
  if (rg == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float yj = alpha * tot[4 + c] + b * tot[8] * e[c];
      y[v_off + c] = io<TOUT>::from_f32(yj);
    }
  }
  float be[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) be[c] = b * e[c];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + RG * m;
    const float ki = sk[i];
    f32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = fmaf(alpha, s[m][c], be[c] * ki);
    __builtin_nontemporal_store(o, reinterpret_cast<f32x4 *>(Su + i * DV + 4 * cg));
  }
}

template <int DK, int DV, typename TIN, typename TOUT>
static hipError_t launch(const DecodeArgs &a) {
  const int units = a.N * a.H;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_step_kernel<DK, DV, TIN, TOUT>), dim3(units), dim3(256), 0,
                     a.stream, static_cast<const TIN *>(a.q), static_cast<const TIN *>(a.k),
                     static_cast<const TIN *>(a.v), a.log_alpha, a.beta, a.A, a.b_alpha, a.S,
                     a.state_idx, a.n_slots, static_cast<TOUT *>(a.y), a.H);
  return hipGetLastError();
}

template <typename TIN, typename TOUT>
static hipError_t launch_d(const DecodeArgs &a) {
  if (a.dk == 128 && a.dv == 128) return launch<128, 128, TIN, TOUT>(a);
  if (a.dk == 128 && a.dv == 64) return launch<128, 64, TIN, TOUT>(a);
  if (a.dk == 64 && a.dv == 128) return launch<64, 128, TIN, TOUT>(a);
  return launch<64, 64, TIN, TOUT>(a);
}

template <typename TIN>
static hipError_t launch_d_out(const DecodeArgs &a) {
  switch (a.out_dtype) {
    case 1: return launch_d<TIN, bf16_t>(a);
    case 2: return launch_d<TIN, _Float16>(a);
    default: return launch_d<TIN, float>(a);
  }
}

hipError_t launch_decode_step(const DecodeArgs &a) {
  switch (a.in_dtype) {
    case 1: return launch_d_out<bf16_t>(a);
    case 2: return launch_d_out<_Float16>(a);
    default: return launch_d_out<float>(a);
  }
}

}  // namespace gdn
