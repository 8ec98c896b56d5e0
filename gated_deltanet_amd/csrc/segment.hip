// Segment-parallel form of the chunked prefill (gfx950).
//
// The state recurrence of the page "NLP——技术报告解读-Qwen3.8-Flash-Next",
// section "Gated DeltaNet 核心机制", is affine in the state: over a stretch of
// tokens, S_out = M S_in + N, where M is the product of the per-token factors
// alpha_t (I - beta_t k_t k_t^T) (a dk x dk matrix: the recurrence run from
// the identity with v = 0) and N is the recurrence run from S_in = 0. Cutting
// a sequence into P segments, the summaries (M_p, N_p) of different segments
// do not depend on each other; a short chain S_in(p + 1) = M_p S_in(p) + N_p
// then gives every segment its true initial state, and each segment after the
// first is run again from it for its outputs. The prefill kernel does all the
// per-segment work (each segment is handed to it as a sequence of a packed
// batch); this file holds the bookkeeping kernels and the chain.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kSegTile = 16;  // state columns per combine workgroup

// Segment bounds of every sequence: segment p of sequence n covers rows
// [bos + min(p L, len), bos + min((p + 1) L, len)) with L = len / P rounded
// up to whole 32-token chunks; cu_seg holds P + 1 bounds per sequence.
__global__ void seg_bounds_kernel(const int32_t *cu, int N, int T, int P, int32_t *cu_seg) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  int64_t bos, len;
  if (cu) {
    int64_t s0 = cu[n], s1 = cu[n + 1];
    s0 = s0 < 0 ? 0 : (s0 > T ? T : s0);
    s1 = s1 < s0 ? s0 : (s1 > T ? T : s1);
    bos = s0;
    len = s1 - s0;
  } else {
    bos = static_cast<int64_t>(n) * T;
    len = T;
  }
  const int64_t L = ((len + P - 1) / P + 31) / 32 * 32;
  for (int p = 0; p <= P; ++p) {
    const int64_t off = static_cast<int64_t>(p) * L;
    cu_seg[static_cast<int64_t>(n) * (P + 1) + p] = static_cast<int32_t>(bos + (off < len ? off : len));
  }
}

// The chain for one sequence, in fp32: Sin[0] = N[0] and
// Sin[e] = M[e - 1] Sin[e - 1] + N[e] for e = 1 .. P - 2 (entry e of Sin is
// the initial state of segment e + 1, of N the zero-start final state of
// segment e, of M the transition of segment e + 1). The columns of the state
// are independent, so one workgroup takes one (head, 16-column tile): 256
// workgroups for 32 heads of 128 columns. The tile of the running state is
// kept transposed in LDS and the head's M row-major; each link's product
// runs on the fp32 matrix cores, and M of the next link is read into
// registers while it runs (M does not depend on the chain).
template <int DK>
__global__ __launch_bounds__(256) void seg_combine_kernel(const float *__restrict__ Nst,
                                                          const float *__restrict__ Mst,
                                                          float *__restrict__ Sin, int H, int DV,
                                                          int P) {
  constexpr int LD = DK + 4;          // padded row length (floats)
  constexpr int NR = DK / 16;         // rows per thread
  constexpr int MV = DK * DK / 4 / 256;  // 16-byte pieces of M per thread
  __shared__ __attribute__((aligned(16))) float St[kSegTile][LD];  // St[j][k] = S[k][j]
  __shared__ __attribute__((aligned(16))) float Ml[DK][LD];
  const int h = blockIdx.x;
  const int j0 = blockIdx.y * kSegTile;
  const int t = threadIdx.x, j = t % kSegTile, i0 = t / kSegTile;
  const size_t st = static_cast<size_t>(H) * DK * DV;
  const size_t mt = static_cast<size_t>(H) * DK * DK;
  auto sidx = [&](int i) { return (static_cast<size_t>(h) * DK + i) * DV + j0 + j; };
  for (int m = 0; m < NR; ++m) {
    const int i = i0 + 16 * m;
    const float v = Nst[sidx(i)];
    St[j][i] = v;
    Sin[sidx(i)] = v;
  }
  if (P <= 2) return;
  f32x4 mreg[MV];
  auto fetch_m = [&](int e) {  // M[e - 1] of this head, 16 bytes per piece
    const f32x4 *M = reinterpret_cast<const f32x4 *>(Mst + (e - 1) * mt +
                                                     static_cast<size_t>(h) * DK * DK);
#pragma unroll
    for (int q = 0; q < MV; ++q) mreg[q] = M[t + 256 * q];
  };
  auto stage_m = [&]() {
#pragma unroll
    for (int q = 0; q < MV; ++q) {
      const int idx = t + 256 * q;  // piece idx: row idx / (DK / 4), columns 4 (idx % (DK / 4))
      *reinterpret_cast<f32x4 *>(&Ml[idx / (DK / 4)][4 * (idx % (DK / 4))]) = mreg[q];
    }
  };
  fetch_m(1);
  stage_m();
  __syncthreads();
  // the product M S on the matrix cores (fp32 16x16x4): wave w forms row
  // tiles w and w + 4 (w + 4 only for DK = 128) of the 16-column result; lane
  // l holds rows 4 (l / 16) + i of its tile, column l % 16
  const int lane = t & 63, wv = t >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  constexpr int TPW = DK / 16 / 4;  // row tiles per wave
  for (int e = 1; e <= P - 2; ++e) {
    if (e + 1 <= P - 2) fetch_m(e + 1);
    f32x4 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = zero4();
#pragma unroll 4
    for (int k0 = 0; k0 < DK; k0 += 4) {
      const float b = St[lr][k0 + lk];  // S[k0 + lk][j0 + lr]
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const float a = Ml[16 * (wv + 4 * u) + lr][k0 + lk];
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[u], 0, 0, 0);
      }
    }
    __syncthreads();  // every read of St and Ml for this link is done
    // plus N, written back transposed for the next link
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * (wv + 4 * u) + 4 * lk + i;
        const size_t o = e * st + (static_cast<size_t>(h) * DK + r) * DV + j0 + lr;
        const float v = acc[u][i] + Nst[o];
        St[lr][r] = v;
        Sin[o] = v;
      }
    if (e + 1 <= P - 2) stage_m();
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_seg_prep(const SegPrepArgs &a) {
  if (a.N > 0)
    hipLaunchKernelGGL(seg_bounds_kernel, dim3((a.N + 255) / 256), dim3(256), 0, a.stream,
                       a.cu_seqlens, a.N, a.T, a.P, a.cu_seg);
  return hipGetLastError();
}

hipError_t launch_seg_combine(const float *Nst, const float *Mst, float *Sin, int H, int dk,
                              int dv, int P, hipStream_t stream) {
  const dim3 grid(H, dv / kSegTile);
  if (dk == 128)
    hipLaunchKernelGGL(seg_combine_kernel<128>, grid, dim3(256), 0, stream, Nst, Mst, Sin, H, dv, P);
  else
    hipLaunchKernelGGL(seg_combine_kernel<64>, grid, dim3(256), 0, stream, Nst, Mst, Sin, H, dv, P);
  return hipGetLastError();
}

}  // namespace gdn
