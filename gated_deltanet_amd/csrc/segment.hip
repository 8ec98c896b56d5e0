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

constexpr int kSegTile = 32;  // state columns per combine workgroup

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

// Initial states of the zero-start runs: segment 0 of each sequence starts
// from the caller's S0 (zeros when absent), the others from zero.
__global__ void seg_s0_kernel(const float *S0, float *S0seg, int N, int nseg, size_t per) {
  const size_t total = static_cast<size_t>(N) * nseg * per;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const size_t x = i % per;
    const size_t e = (i / per) % nseg;
    const size_t n = i / (per * nseg);
    S0seg[i] = (e == 0 && S0) ? S0[n * per + x] : 0.0f;
  }
}

// count identity matrices of size dk x dk
__global__ void seg_ident_kernel(float *I, size_t count, int dk) {
  const size_t per = static_cast<size_t>(dk) * dk;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count * per;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const size_t x = i % per;
    I[i] = (x / dk == x % dk) ? 1.0f : 0.0f;
  }
}

__global__ void seg_zero_kernel(u32x4 *p, size_t n16) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = z;
}

// The chain for one sequence, in fp32: Sin[0] = N[0] and
// Sin[e] = M[e - 1] Sin[e - 1] + N[e] for e = 1 .. P - 2 (entry e of Sin is
// the initial state of segment e + 1, of N the zero-start final state of
// segment e, of M the transition of segment e + 1). One workgroup per (head,
// 32-column tile); the tile of the running state and the head's M stay in
// LDS, each thread owns one column and DK / 8 rows.
template <int DK>
__global__ __launch_bounds__(256) void seg_combine_kernel(const float *__restrict__ Nst,
                                                          const float *__restrict__ Mst,
                                                          float *__restrict__ Sin, int H, int DV,
                                                          int P) {
  __shared__ float Sl[DK][kSegTile + 1];
  __shared__ float Ml[DK][DK + 1];
  const int h = blockIdx.x;
  const int j0 = blockIdx.y * kSegTile;
  const int t = threadIdx.x, j = t % kSegTile, i0 = t / kSegTile;
  constexpr int RS = 256 / kSegTile;  // row stride
  const size_t st = static_cast<size_t>(H) * DK * DV;
  const size_t mt = static_cast<size_t>(H) * DK * DK;
  auto sidx = [&](int i) { return (static_cast<size_t>(h) * DK + i) * DV + j0 + j; };
  for (int i = i0; i < DK; i += RS) {
    const float v = Nst[sidx(i)];
    Sl[i][j] = v;
    Sin[sidx(i)] = v;
  }
  for (int e = 1; e <= P - 2; ++e) {
    const float *M = Mst + (e - 1) * mt + static_cast<size_t>(h) * DK * DK;
    for (int idx = t; idx < DK * DK; idx += 256) Ml[idx / DK][idx % DK] = M[idx];
    __syncthreads();
    float acc[DK / RS];
#pragma unroll
    for (int m = 0; m < DK / RS; ++m) acc[m] = Nst[e * st + sidx(i0 + RS * m)];
    for (int k = 0; k < DK; ++k) {
      const float s = Sl[k][j];
#pragma unroll
      for (int m = 0; m < DK / RS; ++m) acc[m] = fmaf(Ml[i0 + RS * m][k], s, acc[m]);
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < DK / RS; ++m) {
      Sl[i0 + RS * m][j] = acc[m];
      Sin[e * st + sidx(i0 + RS * m)] = acc[m];
    }
    __syncthreads();
  }
}

unsigned grid_for(size_t n, unsigned cap = 4096) {
  const size_t g = (n + 255) / 256;
  return static_cast<unsigned>(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_seg_prep(const SegPrepArgs &a) {
  if (a.N > 0) {
    hipLaunchKernelGGL(seg_bounds_kernel, dim3((a.N + 255) / 256), dim3(256), 0, a.stream,
                       a.cu_seqlens, a.N, a.T, a.P, a.cu_seg);
    const size_t per = static_cast<size_t>(a.H) * a.dk * a.dv;
    const size_t n_s0 = static_cast<size_t>(a.N) * (a.P - 1) * per;
    hipLaunchKernelGGL(seg_s0_kernel, dim3(grid_for(n_s0)), dim3(256), 0, a.stream, a.S0,
                       a.S0seg, a.N, a.P - 1, per);
  }
  if (a.n_ident > 0)
    hipLaunchKernelGGL(seg_ident_kernel, dim3(grid_for(a.n_ident * a.dk * a.dk)), dim3(256), 0,
                       a.stream, a.ident, a.n_ident, a.dk);
  if (a.vzero_bytes > 0)
    hipLaunchKernelGGL(seg_zero_kernel, dim3(grid_for(a.vzero_bytes / 16)), dim3(256), 0,
                       a.stream, static_cast<u32x4 *>(a.vzero), a.vzero_bytes / 16);
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
