// Front end and output gate of the GDN token mixer (gfx950).
//
// Front end (page "NLP——技术报告解读-Qwen3.8-Flash-Next", section
// "GDN 参数化细节", first display; the pwwt.cn page's Fig. 2 caption calls the
// convolution short and causal): for each projected stream and channel c,
//     u_t[c] = sum_{j=0..3} w[c][j] * x_{t-3+j}[c]     (zero before the
//              sequence start, no bias)
//     a_t    = SiLU(u_t)
//     q_t, k_t = a_t / sqrt(sum_c a_t[c]^2 + eps)  per (token, head);  v_t = a_t.
// Output gate (same section, third display; zero-centred RMSNorm from the
// pwwt.cn page, section 2.1.1): per (token, head) row of dv values
//     o = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + w).
//
// Both are pure HBM streams (~2 flops per byte): one pass over the inputs, one
// over the outputs. A row of 8*G channels is owned by G consecutive lanes
// with 16-byte accesses (8 channels each); the per-row reductions are lane
// shuffles inside those G lanes. The convolution re-reads the three previous
// rows, which are in cache (the same workgroup reads them as its own rows).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kTaps = 4;
constexpr int kRowsPerBlock = 64;

template <typename T>
struct Vec8;
template <>
struct Vec8<float> {
  __device__ static void load(const float *p, float *o) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = a[i];
      o[4 + i] = b[i];
    }
  }
  __device__ static void store(float *p, const float *v) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = v[i];
      b[i] = v[4 + i];
    }
    *reinterpret_cast<f32x4 *>(p) = a;
    *reinterpret_cast<f32x4 *>(p + 4) = b;
  }
};
template <>
struct Vec8<_Float16> {
  __device__ static void load(const _Float16 *p, float *o) { io<_Float16>::load16(p, o); }
  __device__ static void store(_Float16 *p, const float *v) {
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (_Float16)v[i];
    *reinterpret_cast<f16x8 *>(p) = r;
  }
};
template <>
struct Vec8<bf16_t> {
  __device__ static void load(const bf16_t *p, float *o) { io<bf16_t>::load16(p, o); }
  __device__ static void store(bf16_t *p, const float *v) {
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    bf16x8_t r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)v[i];  // round to nearest even
    *reinterpret_cast<bf16x8_t *>(p) = r;
  }
};

// sum over the G consecutive lanes that own one row (G a power of two <= 16)
template <int G>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int off = 1; off < G; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// first row of the sequence containing `row` (rows of a packed batch)
__device__ __forceinline__ int64_t seq_begin(const int32_t *cu, int N, int T, int64_t row) {
  if (!cu) return (row / T) * T;
  int lo = 0, hi = N;  // invariant: cu[lo] <= row < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid;
    else hi = mid;
  }
  const int64_t b = cu[lo];
  return b < 0 ? 0 : b;  // malformed offsets must not address before the buffer
}

// grid: x = row blocks, y = head, z = stream (0 q, 1 k, 2 v)
template <int D, typename TIN, typename TOUT>
__global__ __launch_bounds__(256) void frontend_kernel(
    const TIN *__restrict__ xq, const TIN *__restrict__ xk, const TIN *__restrict__ xv,
    const float *__restrict__ conv_w, const int32_t *__restrict__ cu, int N, int T, int64_t rows,
    int H, float eps, TOUT *__restrict__ oq, TOUT *__restrict__ ok, TOUT *__restrict__ ov) {
  constexpr int G = D / 8;          // lanes per row
  constexpr int RPP = 256 / G;      // rows per pass
  const int s = blockIdx.z;
  const int h = blockIdx.y;
  const TIN *x = s == 0 ? xq : (s == 1 ? xk : xv);
  TOUT *out = s == 0 ? oq : (s == 1 ? ok : ov);
  const bool l2 = s < 2;
  const int g = threadIdx.x % G;
  const int c0 = 8 * g;
  // this lane's taps: 8 channels x 4 taps
  float w[8][kTaps];
  const float *wp = conv_w + (static_cast<size_t>(s) * H * D + static_cast<size_t>(h) * D + c0) * kTaps;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const f32x4 t4 = *reinterpret_cast<const f32x4 *>(wp + c * kTaps);
#pragma unroll
    for (int j = 0; j < kTaps; ++j) w[c][j] = t4[j];
  }
  const int64_t rstride = static_cast<int64_t>(H) * D;
  for (int pass = 0; pass < kRowsPerBlock / RPP; ++pass) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + pass * RPP + threadIdx.x / G;
    const bool live = r < rows;
    const int64_t rr = live ? r : rows - 1;  // keep every lane in the shuffles
    const int64_t bos = seq_begin(cu, N, T, rr);
    float u[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) u[c] = 0.0f;
#pragma unroll
    for (int j = 0; j < kTaps; ++j) {
      const int64_t src = rr - (kTaps - 1) + j;
      if (src >= bos) {
        float xv8[8];
        Vec8<TIN>::load(x + src * rstride + static_cast<int64_t>(h) * D + c0, xv8);
#pragma unroll
        for (int c = 0; c < 8; ++c) u[c] = fmaf(w[c][j], xv8[c], u[c]);
      }
    }
    float a[8], ss = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      a[c] = u[c] / (1.0f + __expf(-u[c]));
      ss = fmaf(a[c], a[c], ss);
    }
    if (l2) {
      const float scale = rsqrtf(row_sum<G>(ss) + eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) a[c] *= scale;
    }
    if (live) Vec8<TOUT>::store(out + rr * rstride + static_cast<int64_t>(h) * D + c0, a);
  }
}

template <int D, typename TIN, typename TZ, typename TOUT>
__global__ __launch_bounds__(256) void output_gate_kernel(const TIN *__restrict__ y,
                                                          const TZ *__restrict__ z,
                                                          const float *__restrict__ nw, float eps,
                                                          TOUT *__restrict__ o, int64_t nrows) {
  constexpr int G = D / 8;
  constexpr int RPP = 256 / G;
  const int g = threadIdx.x % G;
  const int c0 = 8 * g;
  float gain[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) gain[c] = 1.0f + (nw ? nw[c0 + c] : 0.0f);
  for (int pass = 0; pass < kRowsPerBlock / RPP; ++pass) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + pass * RPP + threadIdx.x / G;
    const bool live = r < nrows;
    const int64_t rr = live ? r : nrows - 1;
    float yv[8], zv[8];
    Vec8<TIN>::load(y + rr * D + c0, yv);
    Vec8<TZ>::load(z + rr * D + c0, zv);
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) ss = fmaf(yv[c], yv[c], ss);
    const float inv = rsqrtf(row_sum<G>(ss) * (1.0f / D) + eps);
    float ov[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) ov[c] = yv[c] * inv * gain[c] / (1.0f + __expf(-zv[c]));
    if (live) Vec8<TOUT>::store(o + rr * D + c0, ov);
  }
}

template <int D, typename TIN, typename TOUT>
hipError_t launch_fe(const FrontendArgs &a) {
  const int64_t blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  dim3 grid(static_cast<unsigned>(blocks), a.H, 3);
  hipLaunchKernelGGL((frontend_kernel<D, TIN, TOUT>), grid, dim3(256), 0, a.stream,
                     static_cast<const TIN *>(a.xq), static_cast<const TIN *>(a.xk),
                     static_cast<const TIN *>(a.xv), a.conv_w, a.cu_seqlens, a.N, a.T, a.rows, a.H,
                     a.eps, static_cast<TOUT *>(a.q), static_cast<TOUT *>(a.k),
                     static_cast<TOUT *>(a.v));
  return hipGetLastError();
}

template <int D, typename TIN, typename TZ, typename TOUT>
hipError_t launch_og(const GateArgs &a) {
  const int64_t blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((output_gate_kernel<D, TIN, TZ, TOUT>), dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, a.stream, static_cast<const TIN *>(a.y),
                     static_cast<const TZ *>(a.z), a.norm_w, a.eps, static_cast<TOUT *>(a.o),
                     a.rows);
  return hipGetLastError();
}

// runtime dtype code (0 f32, 1 bf16, 2 f16) -> type, one template level at a time
template <typename F>
hipError_t with_type(int code, F &&f) {
  switch (code) {
    case 1: return f(bf16_t{});
    case 2: return f(_Float16{});
    default: return f(float{});
  }
}

}  // namespace

hipError_t launch_frontend(const FrontendArgs &a) {
  if (a.rows == 0) return hipSuccess;
  return with_type(a.in_dtype, [&](auto tin) {
    return with_type(a.out_dtype, [&](auto tout) {
      using TI = decltype(tin);
      using TO = decltype(tout);
      return a.d == 128 ? launch_fe<128, TI, TO>(a) : launch_fe<64, TI, TO>(a);
    });
  });
}

hipError_t launch_output_gate(const GateArgs &a) {
  if (a.rows == 0) return hipSuccess;
  return with_type(a.in_dtype, [&](auto ty) {
    return with_type(a.z_dtype, [&](auto tz) {
      return with_type(a.out_dtype, [&](auto to) {
        using TY = decltype(ty);
        using TZ = decltype(tz);
        using TO = decltype(to);
        return a.d == 128 ? launch_og<128, TY, TZ, TO>(a) : launch_og<64, TY, TZ, TO>(a);
      });
    });
  });
}

}  // namespace gdn
