// common.hpp - shared device helpers for the gfx950 TANGO/WANGO kernels.
//
// MFMA fragments.  Every matrix product in the library is built from 16x16
// output blocks.  A lane l of a 64-wide wavefront holds, for an A operand, row
// (l % 16) and eight k-slots of lane group g = l / 16; for a B operand, column
// (l % 16) and the same eight k-slots of group g.  The accumulator block holds
// column (l % 16) and rows 4g + r, r = 0..3.
//
// Which k index a (group, slot) pair stands for only has to agree between the
// A and the B operand of one product, so each kernel picks the assignment that
// makes its loads contiguous.  Two are used:
//   * "linear":   slot s of group g is k = 8g + s;
//   * "permuted": slot s of group g is k = 4g + s for s < 4 and 16 + 4g + (s-4)
//                 for s >= 4.  It is the row order of two stacked accumulator
//                 blocks, so an accumulator pair can feed the next product
//                 directly, and it is the order of the packed gate layout.
//
// bf16 products use v_mfma_f32_16x16x32_bf16 (one instruction per fragment).
// fp32 products use eight v_mfma_f32_16x16x4_f32, slot s of every lane group
// going into instruction s, which visits the same (group, slot) -> k pairs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tango {

typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <typename T> struct Vec;
template <> struct Vec<bf16> {
  using frag = bf16x8;   // 8 elements, 16 bytes
  using quad = bf16x4;   // 4 elements, 8 bytes
};
template <> struct Vec<float> {
  using frag = f32x8;    // 8 elements, 32 bytes
  using quad = f32x4;    // 4 elements, 16 bytes
};
template <typename T> using Frag = typename Vec<T>::frag;
template <typename T> using Quad = typename Vec<T>::quad;

__device__ __forceinline__ void mma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 join(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x8 join(const f32x4& lo, const f32x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// float -> storage type, round to nearest even.
template <typename T> __device__ __forceinline__ T cvt(float x);
template <> __device__ __forceinline__ bf16 cvt<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float cvt<float>(float x) { return x; }

template <typename T> __device__ __forceinline__ float tof(T x) { return (float)x; }

template <typename T> __device__ __forceinline__ Quad<T> cvt_quad(const f32x4& v) {
  Quad<T> q;
#pragma unroll
  for (int r = 0; r < 4; ++r) q[r] = cvt<T>(v[r]);
  return q;
}

template <typename T> __device__ __forceinline__ f32x4 quad_to_f32(const Quad<T>& q) {
  f32x4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = tof<T>(q[r]);
  return v;
}

template <typename T> __device__ __forceinline__ Frag<T> load_frag(const T* p) {
  return *reinterpret_cast<const Frag<T>*>(p);
}
template <typename T> __device__ __forceinline__ Quad<T> load_quad(const T* p) {
  return *reinterpret_cast<const Quad<T>*>(p);
}
template <typename T> __device__ __forceinline__ void store_quad(T* p, const Quad<T>& q) {
  *reinterpret_cast<Quad<T>*>(p) = q;
}
template <typename T> __device__ __forceinline__ void store_frag(T* p, const Frag<T>& f) {
  *reinterpret_cast<Frag<T>*>(p) = f;
}

// Source order of the packed gate layout and of the "permuted" k-slots:
// slot s of lane group g within a block of 32 positions.
__host__ __device__ __forceinline__ int perm_slot(int g, int s) {
  return s < 4 ? 4 * g + s : 16 + 4 * g + (s - 4);
}

// Position of feature e (0..31 within a group of 32) in the permuted feature
// order: slot s of lane group g holds feature perm_slot(g, s), stored at 8g + s.
__host__ __device__ __forceinline__ int feature_slot(int e32) {
  return e32 < 16 ? (e32 >> 2) * 8 + (e32 & 3) : ((e32 - 16) >> 2) * 8 + 4 + (e32 & 3);
}

// WANGO positive feature map phi(u) = max(ELU(u) + 1 + 1e-4, 1e-4) / sqrt(d_h)
// ([TANGO] §2.2 eq. 8), ELU with alpha = 1; inv_sqrt_dh = 1 / sqrt(d_h).
__device__ __forceinline__ float phi_feature(float u, float inv_sqrt_dh) {
  const float elu1 = u > 0.f ? u + 1.0f : __expf(u);   // ELU(u) + 1
  return fmaxf(elu1 + 1e-4f, 1e-4f) * inv_sqrt_dh;
}

// Offset (in elements) of g[row m, column f] in the packed gate layout
// [M/32][4][F][8], M = all (batch, padded position) rows.
__host__ __device__ __forceinline__ int64_t packed_offset(int64_t blk, int grp, int64_t f,
                                                          int64_t F) {
  return ((blk * 4 + grp) * F + f) * 8;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over lanes that share l % 16 (the four lane groups).
__device__ __forceinline__ float group_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace tango
