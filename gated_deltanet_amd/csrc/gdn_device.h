// Device-side helpers shared by the libgdn kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 is carried as its 16 raw bits.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round to nearest even; NaN stays NaN (quiet bit forced)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Element-type traits for global inputs and outputs.
template <typename T>
struct io;

template <>
struct io<float> {
  static constexpr int kVec = 4;  // elements per 16-byte access
  __device__ static __forceinline__ void load16(const float *p, float *out) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
    out[0] = v[0];
    out[1] = v[1];
    out[2] = v[2];
    out[3] = v[3];
  }
  __device__ static __forceinline__ float to_f32(float x) { return x; }
  __device__ static __forceinline__ float from_f32(float x) { return x; }
};

template <>
struct io<bf16_t> {
  static constexpr int kVec = 8;
  __device__ static __forceinline__ void load16(const bf16_t *p, float *out) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }
  __device__ static __forceinline__ bf16_t from_f32(float x) { return f32_to_bf16(x); }
};

template <>
struct io<_Float16> {
  static constexpr int kVec = 8;
  __device__ static __forceinline__ void load16(const _Float16 *p, float *out) {
    const f16x8 v = *reinterpret_cast<const f16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = static_cast<float>(v[i]);
  }
  __device__ static __forceinline__ float to_f32(_Float16 x) { return static_cast<float>(x); }
  __device__ static __forceinline__ _Float16 from_f32(float x) { return static_cast<_Float16>(x); }
};

// ---------------------------------------------------------------------------
// MFMA fragments.
//
// All products use the 16x16 output tile of the gfx950 matrix cores. A lane
// l = 16*lg + lc of a wave owns, in an accumulator tile, rows 4*lg + i
// (i = 0..3) of column lc. A "fragment" is the lane's share of a 32-deep
// slice of an operand: 8 values, for row (A) or column (B) index lc, at the
// contraction indices
//     slot j < 4 : 4*lg + j          slot j >= 4 : 16 + 4*lg + (j - 4)
// within the slice. Because the hardware sums slot-by-slot over the lanes of
// one row/column, any bijection between slots and contraction indices that
// A and B share gives the same product; this one makes the two accumulator
// tiles that cover rows 0..15 and 16..31 of a 32-row block directly usable
// as a B fragment (slots 0-3 from the first tile, 4-7 from the second), so
// results chain into the next product without a trip through LDS.
// ---------------------------------------------------------------------------

template <typename MT>
struct Frag;

// fp16 operands: one v_mfma_f32_16x16x32_f16 per fragment pair.
template <>
struct Frag<_Float16> {
  f16x8 v;
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (_Float16)0.0f;
  }
  // from two accumulator tiles (rows 0..15 and 16..31 of the slice)
  __device__ __forceinline__ void from_acc(const f32x4 &a, const f32x4 &b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = (_Float16)a[j];
      v[4 + j] = (_Float16)b[j];
    }
  }
  __device__ __forceinline__ void from_acc_lo(const f32x4 &a) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = (_Float16)a[j];
      v[4 + j] = (_Float16)0.0f;
    }
  }
  // row-major LDS matrix, row `row`, slice starting at column c0
  __device__ __forceinline__ void load_row(const _Float16 *base, int ld, int row, int c0,
                                           int lg) {
    const _Float16 *p = base + row * ld + c0 + 4 * lg;
    const f16x4 a = *reinterpret_cast<const f16x4 *>(p);
    const f16x4 b = *reinterpret_cast<const f16x4 *>(p + 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  }
  // same, but contraction indices >= 16 of the slice are taken as zero
  __device__ __forceinline__ void load_row_lo(const _Float16 *base, int ld, int row, int c0,
                                              int lg) {
    const _Float16 *p = base + row * ld + c0 + 4 * lg;
    const f16x4 a = *reinterpret_cast<const f16x4 *>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = (_Float16)0.0f;
    }
  }
  // row-major fp32 LDS matrix, converted
  __device__ __forceinline__ void load_row_f32(const float *base, int ld, int row, int c0,
                                               int lg) {
    const float *p = base + row * ld + c0 + 4 * lg;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = (_Float16)a[j];
      v[4 + j] = (_Float16)b[j];
    }
  }
  // column `col` of a row-major LDS matrix, slice starting at row r0
  __device__ __forceinline__ void load_col(const _Float16 *base, int ld, int col, int r0,
                                           int lg) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = base[(r0 + 4 * lg + j) * ld + col];
      v[4 + j] = base[(r0 + 16 + 4 * lg + j) * ld + col];
    }
  }
  __device__ __forceinline__ void load_col_lo(const _Float16 *base, int ld, int col, int r0,
                                              int lg) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = base[(r0 + 4 * lg + j) * ld + col];
      v[4 + j] = (_Float16)0.0f;
    }
  }
};

// fp32 operands: eight v_mfma_f32_16x16x4_f32 per fragment pair (slot j is
// the lane's single contraction value of instruction j).
template <>
struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  }
  __device__ __forceinline__ void from_acc(const f32x4 &a, const f32x4 &b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  }
  __device__ __forceinline__ void from_acc_lo(const f32x4 &a) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = 0.0f;
    }
  }
  __device__ __forceinline__ void load_row(const float *base, int ld, int row, int c0, int lg) {
    const float *p = base + row * ld + c0 + 4 * lg;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  }
  __device__ __forceinline__ void load_row_lo(const float *base, int ld, int row, int c0,
                                              int lg) {
    const float *p = base + row * ld + c0 + 4 * lg;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = 0.0f;
    }
  }
  __device__ __forceinline__ void load_row_f32(const float *base, int ld, int row, int c0,
                                               int lg) {
    load_row(base, ld, row, c0, lg);
  }
  __device__ __forceinline__ void load_col(const float *base, int ld, int col, int r0, int lg) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = base[(r0 + 4 * lg + j) * ld + col];
      v[4 + j] = base[(r0 + 16 + 4 * lg + j) * ld + col];
    }
  }
  __device__ __forceinline__ void load_col_lo(const float *base, int ld, int col, int r0,
                                              int lg) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = base[(r0 + 4 * lg + j) * ld + col];
      v[4 + j] = 0.0f;
    }
  }
};

// acc += A_slice * B_slice (16x32 times 32x16)
__device__ __forceinline__ void mma(f32x4 &acc, const Frag<_Float16> &a,
                                    const Frag<_Float16> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  return z;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// sum over the G consecutive lanes that own one row (G = 8 or 16: a half or a
// whole 16-lane DPP row): pairs and quads by quad permutes, then quads joined
// by the half-row and row mirrors; every lane ends with the row's sum
template <int G>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(G == 8 || G == 16, "row width");
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  if constexpr (G == 16) v += dpp<0x140>(v);  // row_mirror
  return v;
}

// Gates from raw per-head pre-activations (page "NLP——技术报告解读-
// Qwen3.8-Flash-Next", section "GDN 参数化细节"): the decay gate is
// alpha = exp(-exp(A) softplus(a + b_alpha)) and the write gate is
// beta = sigmoid(b). RawGate holds exp(A) and b_alpha of one head; scale = 0
// marks gates that arrive already as log alpha and beta.
struct RawGate {
  float scale;  // exp(A_h), or 0 when the gates are not raw
  float bias;   // b_alpha of the head

  __device__ static __forceinline__ RawGate load(const float *A, const float *b_alpha, int h) {
    RawGate g{0.0f, 0.0f};
    if (A) {
      g.scale = expf(A[h]);
      if (b_alpha) g.bias = b_alpha[h];
    }
    return g;
  }
  __device__ __forceinline__ bool raw() const { return scale != 0.0f; }
  // softplus(x) = max(x, 0) + log(1 + exp(-|x|)), accurate at both ends
  __device__ __forceinline__ float log_alpha(float a) const {
    const float x = a + bias;
    return -scale * (fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))));
  }
  __device__ static __forceinline__ float beta(float b) { return 1.0f / (1.0f + expf(-b)); }
};

}  // namespace gdn
