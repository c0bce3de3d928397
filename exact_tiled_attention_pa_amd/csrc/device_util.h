// Device-side helpers shared by the gfx950 kernels: bf16 packing, DPP row
// reductions, vector types for MFMA operands.  Internal header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// bf16 bit patterns packed two per 32-bit word: element 2i in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> bf16x2 word, round to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// DPP lane moves inside a 16-lane row.
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of LANES consecutive lanes (LANES = 8 or 16); every lane of a
// group ends with the same (bitwise) value.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 8 || LANES == 16, "group of 8 or 16 lanes");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  if constexpr (LANES == 16) x += dpp<kDppRowMirror>(x);
  return x;
}

// Reductions over the lane pair (l, l ^ 32).  v_permlane32_swap exchanges the
// upper half of its destination with the lower half of its source; called with
// the same value in both, the two results hold x[l] and x[l ^ 32] in some order
// in every lane, so the symmetric combination below is the pair reduction.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                            false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                            false);
  // IEEE addition is commutative, so both lanes of a pair get the same bits
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Decode grids are (columns, rows, sequence) with many rows past a short sequence's
// last split.  The hardware deals a kernel's workgroups to the shader engines of an XCD
// in launch order, round robin, and dispatches them in order, so an engine that keeps
// receiving the costly low rows paces its whole XCD while the others idle.  Rotating
// each sequence's rows (and columns) by its index spreads every sequence's live splits
// evenly over the engines; it is a bijection per sequence, so each split is still
// computed by exactly one workgroup.
__device__ __forceinline__ int rotated_grid_index(int i, int n, int seq) {
  return (int)(((unsigned)i + (unsigned)seq) % (unsigned)n);
}

// Split walked by grouped-head decode grid row y (see decode_grid_splits): with a
// sliding window the rows count back from the sequence's last split, else row y is
// split y.  Negative: nothing to do.
__device__ __forceinline__ int decode_split_of(int y, int seq_len, int split_tokens,
                                               int window) {
  return window > 0 ? (seq_len > 0 ? (seq_len - 1) / split_tokens : 0) - y : y;
}

// Factor applied to raw q.k dot products: scale * log2(e), so that softmax
// weights are exp2(s * c - m).  A zero scale is raised to the smallest normal
// float: every finite score then maps to exactly exp2(0) = 1 (uniform weights,
// the exact answer for scale 0), while a masked -inf score stays -inf instead of
// becoming -inf * 0 = NaN.
inline float score_scale_log2(float scale) {
  const float c = scale * kLog2e;
  return c < 1.17549435e-38f ? 1.17549435e-38f : c;
}

}  // namespace pa
