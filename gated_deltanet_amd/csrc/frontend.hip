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
// with 16-byte accesses (8 channels each); the per-row reductions are DPP
// lane exchanges inside those G lanes. The front end streams whole rows down a
// block of tokens and keeps the three previous rows of its channels in
// registers for the causal taps, so every input byte is read from memory
// about once.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kTaps = 4;
constexpr int kRowsPerBlock = 64;  // output gate rows per workgroup

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

// 1 / (1 + exp(-x)) with one v_exp_f32 and one v_rcp_f32 (about 1 ulp each);
// exp overflows to inf for x < -88 and the reciprocal then gives 0
__device__ __forceinline__ float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// index of the sequence containing `row` of a packed batch: the last k with
// cu[k] <= row (0 if none). Called with a row that is uniform across the
// workgroup, so the loads go through the scalar cache.
__device__ __forceinline__ int seq_index(const int32_t *cu, int N, int64_t row) {
  int lo = 0, hi = N;  // invariant: cu[lo] <= row < cu[hi] (when well formed)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Eight elements of type T as raw bits in registers (16 bytes for 16-bit
// types, 32 for fp32).
template <typename T>
struct Raw8 {
  u32x4 v[sizeof(T) / 2];
};
template <typename T>
__device__ __forceinline__ Raw8<T> load_raw8(const T *p) {
  Raw8<T> r;
#pragma unroll
  for (int q = 0; q < static_cast<int>(sizeof(T)) / 2; ++q)
    r.v[q] = reinterpret_cast<const u32x4 *>(p)[q];
  return r;
}
__device__ __forceinline__ void raw8_to_f32(const Raw8<float> &r, float *o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = __uint_as_float(r.v[0][i]);
    o[4 + i] = __uint_as_float(r.v[1][i]);
  }
}
__device__ __forceinline__ void raw8_to_f32(const Raw8<bf16_t> &r, float *o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(r.v[0][i] << 16);
    o[2 * i + 1] = __uint_as_float(r.v[0][i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void raw8_to_f32(const Raw8<_Float16> &r, float *o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(r.v[0][i])));
    o[2 * i + 1] =
        static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(r.v[0][i] >> 16)));
  }
}

constexpr int kFeRows = 64;   // rows per workgroup, streamed in order
constexpr int kFeAhead = 8;   // rows of loads in flight per lane

// One workgroup streams kFeRows consecutive rows of one stream (0 q, 1 k,
// 2 v); its lanes cover (head, 8-channel group) pairs, 256 per workgroup
// (grid.y covers the rest), so a row is read and written as one contiguous
// span. The three previous rows of each lane's channels stay in registers
// and are cleared at every sequence start (uniform bookkeeping).
// grid: x = stream * row_blocks + row_block, y = slice of the H*D/8 pairs
template <int D, typename TIN, typename TOUT>
__global__ __launch_bounds__(256) void frontend_kernel(
    const TIN *__restrict__ xq, const TIN *__restrict__ xk, const TIN *__restrict__ xv,
    const float *__restrict__ conv_w, const int32_t *__restrict__ cu, int N, int T, int64_t rows,
    int H, float eps, TOUT *__restrict__ oq, TOUT *__restrict__ ok, TOUT *__restrict__ ov) {
  constexpr int G = D / 8;  // lanes per (token, head) row
  const int64_t nrb = (rows + kFeRows - 1) / kFeRows;
  const int s = static_cast<int>(blockIdx.x / nrb);
  const int64_t rb = blockIdx.x % nrb;
  const int hg = blockIdx.y * 256 + threadIdx.x;
  const bool active = hg < H * G;
  const int hgc = active ? hg : 0;  // idle lanes shadow pair 0 (in bounds, never stored)
  const TIN *x = s == 0 ? xq : (s == 1 ? xk : xv);
  TOUT *out = s == 0 ? oq : (s == 1 ? ok : ov);
  const bool l2 = s < 2;
  const int64_t col = static_cast<int64_t>(hgc) * 8;  // = head * D + 8 * group
  float w[8][kTaps];
  const float *wp = conv_w + (static_cast<size_t>(s) * H * D + col) * kTaps;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const f32x4 t4 = *reinterpret_cast<const f32x4 *>(wp + c * kTaps);
#pragma unroll
    for (int j = 0; j < kTaps; ++j) w[c][j] = t4[j];
  }
  const int64_t rstride = static_cast<int64_t>(H) * D;
  const int64_t r_first = rb * kFeRows;
  const int64_t r_end = r_first + kFeRows < rows ? r_first + kFeRows : rows;
  // current sequence [bos, next); uniform across the workgroup
  int k = 0;
  int64_t bos, next;
  if (cu) {
    k = seq_index(cu, N, r_first);
    bos = cu[k];
    next = cu[k + 1];
  } else {
    bos = (r_first / T) * T;
    next = bos + T;
  }
  auto advance = [&](int64_t row) {  // move [bos, next) to the sequence holding row
    while (row >= next) {
      if (cu) {
        if (k + 1 >= N) {
          bos = next;
          next = INT64_MAX;
          break;
        }
        ++k;
        bos = next;
        next = cu[k + 1];
      } else {
        bos = next;
        next += T;
      }
    }
  };
  // the three rows before r_first, zero outside the sequence of r_first
  float x1[8], x2[8], x3[8];
  {
    float* win[3] = {x1, x2, x3};
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int64_t row = r_first - 1 - j;
      if (row >= bos && row >= 0) {
        raw8_to_f32(load_raw8(x + row * rstride + col), win[j]);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) win[j][c] = 0.0f;
      }
    }
  }
  Raw8<TIN> buf[kFeAhead];
#pragma unroll
  for (int i = 0; i < kFeAhead; ++i)
    if (r_first + i < r_end) buf[i] = load_raw8(x + (r_first + i) * rstride + col);
#pragma unroll 1
  for (int64_t r0 = r_first; r0 < r_end; r0 += kFeAhead) {
#pragma unroll
    for (int i = 0; i < kFeAhead; ++i) {
      const int64_t row = r0 + i;
      if (row >= r_end) break;
      float xc[8];
      raw8_to_f32(buf[i], xc);
      if (row + kFeAhead < r_end) buf[i] = load_raw8(x + (row + kFeAhead) * rstride + col);
      if (row >= next) {
        advance(row);
        if (row == bos) {
#pragma unroll
          for (int c = 0; c < 8; ++c) x1[c] = x2[c] = x3[c] = 0.0f;
        }
      }
      float a[8], ss = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float u = w[c][3] * xc[c] + w[c][2] * x1[c] + w[c][1] * x2[c] + w[c][0] * x3[c];
        a[c] = u * sigmoid(u);
        ss = fmaf(a[c], a[c], ss);
        x3[c] = x2[c];
        x2[c] = x1[c];
        x1[c] = xc[c];
      }
      if (l2) {
        const float scale = rsqrtf(row_sum<G>(ss) + eps);
#pragma unroll
        for (int c = 0; c < 8; ++c) a[c] *= scale;
      }
      if (active) Vec8<TOUT>::store(out + row * rstride + col, a);
    }
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
    for (int c = 0; c < 8; ++c) ov[c] = yv[c] * inv * gain[c] * sigmoid(zv[c]);
    if (live) Vec8<TOUT>::store(o + rr * D + c0, ov);
  }
}

template <int D, typename TIN, typename TOUT>
hipError_t launch_fe(const FrontendArgs &a) {
  const int64_t blocks = (a.rows + kFeRows - 1) / kFeRows * 3;
  const int slices = (a.H * (D / 8) + 255) / 256;
  hipLaunchKernelGGL((frontend_kernel<D, TIN, TOUT>), dim3(static_cast<unsigned>(blocks), slices),
                     dim3(256), 0, a.stream, static_cast<const TIN *>(a.xq),
                     static_cast<const TIN *>(a.xk), static_cast<const TIN *>(a.xv), a.conv_w,
                     a.cu_seqlens, a.N, a.T, a.rows, a.H, a.eps, static_cast<TOUT *>(a.q),
                     static_cast<TOUT *>(a.k), static_cast<TOUT *>(a.v));
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

// Convolution cache after a prefill: for each sequence, head and stream the
// last three raw rows, oldest first, zeros where the sequence is shorter;
// a plain copy of the raw bits (element type E of the raw projections).
template <typename E>
__global__ __launch_bounds__(256) void conv_state_kernel(const ConvStateArgs a) {
  const int n = blockIdx.x / a.H;
  const int h = blockIdx.x % a.H;
  const int slot = a.slot_idx ? a.slot_idx[n] : n;
  if (slot < 0 || slot >= a.n_slots) return;
  int64_t bos, len;
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
  const E *src[3] = {static_cast<const E *>(a.xq), static_cast<const E *>(a.xk),
                     static_cast<const E *>(a.xv)};
  E *dst = static_cast<E *>(a.conv_state) + (static_cast<size_t>(slot) * a.H + h) * 9 * a.d;
  for (int idx = threadIdx.x; idx < 9 * a.d; idx += 256) {
    const int s = idx / (3 * a.d);      // stream
    const int r = (idx / a.d) % 3;      // 0 = oldest
    const int c = idx % a.d;
    const int64_t t = len - 3 + r;      // row inside the sequence
    dst[idx] = t >= 0 ? src[s][((bos + t) * a.H + h) * a.d + c] : E(0);
  }
}

hipError_t launch_conv_state(const ConvStateArgs &a) {
  const int64_t blocks = static_cast<int64_t>(a.N) * a.H;
  if (blocks == 0) return hipSuccess;
  if (a.elem_bytes == 4)
    hipLaunchKernelGGL(conv_state_kernel<uint32_t>, dim3(static_cast<unsigned>(blocks)), dim3(256),
                       0, a.stream, a);
  else
    hipLaunchKernelGGL(conv_state_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256),
                       0, a.stream, a);
  return hipGetLastError();
}

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
