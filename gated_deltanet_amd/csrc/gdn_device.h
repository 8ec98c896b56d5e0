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
// the same for a 16-deep slice (slots 4..7 zero): half the instructions
__device__ __forceinline__ void mma_lo(f32x4 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  return z;
}

// Unit lower-triangular solve of one 16x16 diagonal block held column-wise
// across a 16-lane DPP row: lane c holds ac[r] = A[r][c] (strictly lower part
// used) and, on entry, xv[r] = the right-hand side of column c (e.g. the
// identity); on exit xv[r] = ((I + A)^-1)[r][c]. Step s subtracts A[r][s] x_s
// from x_r for r > s, with A[r][s] broadcast from lane s of the row by
// v_fmac_f32_dpp row_newbcast:s (so A is never re-read from memory). The
// leading s_nop of each step gives the two wait states a DPP source needs
// after a VALU write (the compiler does not guard inline asm).
__device__ __forceinline__ void unit_lower_solve16(const float *ac, float *xv) {
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%15, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%16, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%17, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%18, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %4, -%19, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %5, -%20, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %6, -%21, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %7, -%22, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %8, -%23, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %9, -%24, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %10, -%25, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %11, -%26, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %12, -%27, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %13, -%28, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %14, -%29, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[1]), "+v"(xv[2]), "+v"(xv[3]), "+v"(xv[4]), "+v"(xv[5]), "+v"(xv[6]), "+v"(xv[7]), "+v"(xv[8]), "+v"(xv[9]), "+v"(xv[10]), "+v"(xv[11]), "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[1]), "v"(ac[2]), "v"(ac[3]), "v"(ac[4]), "v"(ac[5]), "v"(ac[6]), "v"(ac[7]), "v"(ac[8]), "v"(ac[9]), "v"(ac[10]), "v"(ac[11]), "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[0]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%14, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%15, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%16, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%17, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %4, -%18, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %5, -%19, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %6, -%20, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %7, -%21, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %8, -%22, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %9, -%23, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %10, -%24, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %11, -%25, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %12, -%26, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %13, -%27, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[2]), "+v"(xv[3]), "+v"(xv[4]), "+v"(xv[5]), "+v"(xv[6]), "+v"(xv[7]), "+v"(xv[8]), "+v"(xv[9]), "+v"(xv[10]), "+v"(xv[11]), "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[2]), "v"(ac[3]), "v"(ac[4]), "v"(ac[5]), "v"(ac[6]), "v"(ac[7]), "v"(ac[8]), "v"(ac[9]), "v"(ac[10]), "v"(ac[11]), "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[1]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%13, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%14, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%15, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%16, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %4, -%17, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %5, -%18, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %6, -%19, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %7, -%20, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %8, -%21, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %9, -%22, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %10, -%23, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %11, -%24, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %12, -%25, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[3]), "+v"(xv[4]), "+v"(xv[5]), "+v"(xv[6]), "+v"(xv[7]), "+v"(xv[8]), "+v"(xv[9]), "+v"(xv[10]), "+v"(xv[11]), "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[3]), "v"(ac[4]), "v"(ac[5]), "v"(ac[6]), "v"(ac[7]), "v"(ac[8]), "v"(ac[9]), "v"(ac[10]), "v"(ac[11]), "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[2]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%12, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%13, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%14, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%15, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %4, -%16, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %5, -%17, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %6, -%18, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %7, -%19, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %8, -%20, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %9, -%21, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %10, -%22, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %11, -%23, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[4]), "+v"(xv[5]), "+v"(xv[6]), "+v"(xv[7]), "+v"(xv[8]), "+v"(xv[9]), "+v"(xv[10]), "+v"(xv[11]), "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[4]), "v"(ac[5]), "v"(ac[6]), "v"(ac[7]), "v"(ac[8]), "v"(ac[9]), "v"(ac[10]), "v"(ac[11]), "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[3]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%11, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%12, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%13, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%14, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %4, -%15, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %5, -%16, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %6, -%17, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %7, -%18, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %8, -%19, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %9, -%20, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %10, -%21, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[5]), "+v"(xv[6]), "+v"(xv[7]), "+v"(xv[8]), "+v"(xv[9]), "+v"(xv[10]), "+v"(xv[11]), "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[5]), "v"(ac[6]), "v"(ac[7]), "v"(ac[8]), "v"(ac[9]), "v"(ac[10]), "v"(ac[11]), "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[4]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%10, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%11, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%12, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%13, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %4, -%14, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %5, -%15, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %6, -%16, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %7, -%17, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %8, -%18, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %9, -%19, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[6]), "+v"(xv[7]), "+v"(xv[8]), "+v"(xv[9]), "+v"(xv[10]), "+v"(xv[11]), "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[6]), "v"(ac[7]), "v"(ac[8]), "v"(ac[9]), "v"(ac[10]), "v"(ac[11]), "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[5]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%9, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%10, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%11, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%12, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %4, -%13, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %5, -%14, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %6, -%15, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %7, -%16, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %8, -%17, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[7]), "+v"(xv[8]), "+v"(xv[9]), "+v"(xv[10]), "+v"(xv[11]), "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[7]), "v"(ac[8]), "v"(ac[9]), "v"(ac[10]), "v"(ac[11]), "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[6]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%8, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%9, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%10, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%11, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %4, -%12, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %5, -%13, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %6, -%14, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %7, -%15, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[8]), "+v"(xv[9]), "+v"(xv[10]), "+v"(xv[11]), "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[8]), "v"(ac[9]), "v"(ac[10]), "v"(ac[11]), "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[7]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%7, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%8, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%9, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%10, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %4, -%11, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %5, -%12, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %6, -%13, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[9]), "+v"(xv[10]), "+v"(xv[11]), "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[9]), "v"(ac[10]), "v"(ac[11]), "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[8]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%6, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%7, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%8, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%9, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %4, -%10, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %5, -%11, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[10]), "+v"(xv[11]), "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[10]), "v"(ac[11]), "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[9]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%5, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%6, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%7, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%8, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %4, -%9, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[11]), "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[11]), "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[10]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%4, %8 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%5, %8 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%6, %8 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, -%7, %8 row_newbcast:11 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[12]), "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[12]), "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[11]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%3, %6 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%4, %6 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, -%5, %6 row_newbcast:12 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[13]), "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[13]), "v"(ac[14]), "v"(ac[15]), "v"(xv[12]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%2, %4 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, -%3, %4 row_newbcast:13 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[14]), "+v"(xv[15])
               : "v"(ac[14]), "v"(ac[15]), "v"(xv[13]));
  asm volatile("s_nop 1\n\t"
               "v_fmac_f32_dpp %0, -%1, %2 row_newbcast:14 row_mask:0xf bank_mask:0xf"
               : "+v"(xv[15])
               : "v"(ac[15]), "v"(xv[14]));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// row_shr:N inside each 16-lane DPP row; lanes without a source read 0
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, true));
}
// value of lane l (uniform)
__device__ __forceinline__ float lane_value(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// inclusive prefix sums over each 32-lane half of the wave: within 16-lane
// rows by DPP shifts, then the second row of each half adds the first's last
__device__ __forceinline__ float scan32(float x, int lane) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  const float r15 = lane_value(x, 15), r47 = lane_value(x, 47);
  if ((lane & 31) >= 16) x += lane < 32 ? r15 : r47;
  return x;
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

// x + (the value of lane ^ 16) and x + (the value of lane ^ 32), by the CDNA4
// lane-swap instructions (VALU, no LDS round trip): v_permlane16_swap trades
// the odd 16-lane rows of its first operand with the even rows of its second,
// v_permlane32_swap the upper half of the first with the lower half of the
// second; with two copies of x the pair then holds both values of every
// lane pair. Written as inline asm since the compiler's builtin returns its
// second result wrongly; the s_nop gives the two wait states a VALU write
// needs before these instructions read it.
__device__ __forceinline__ float xor16_sum(float x) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}
__device__ __forceinline__ float xor32_sum(float x) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
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

// Chunk-start states handed from the prefill kernel to the backward pass.
// A 32-column tile of one state is kept by two waves, each owning a 16-column
// slab as dk/16 accumulator tiles; element i of tile t in lane (lg, lc) is
// state row state_row(t, lg, i) (the key order of the fragment-linear K and
// Q slices), column 16 * slab + lc. The workspace stores each such f32x4 as
// it sits in the lane: per (chunk slot, head, column tile) a block of
// dk x 32 floats ordered [slab][t][lane][i], so every store and load is one
// coalesced 16-byte access per lane.
__device__ __forceinline__ int state_row(int t, int lg, int i) {
  return 32 * (t >> 1) + 8 * lg + 4 * (t & 1) + i;
}

}  // namespace gdn
