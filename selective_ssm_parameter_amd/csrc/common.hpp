// Shared device helpers for the Swimba kernels (gfx950 / CDNA4).
//
// Matrix-core convention used throughout: a 16x16 output tile is computed by
// one 64-lane wave. Lane l belongs to lane group g = l / 16 and column (or row)
// c = l % 16. An operand "fragment" is 8 consecutive contraction elements per
// lane: for the A operand, lane l holds A[c][k-slots of group g]; for the B
// operand, lane l holds B[k-slots of group g][c]. A and B always use the same
// mapping from (group, element) to the contraction index, so the contraction
// may visit k in any order we choose. The fp32 accumulator tile D holds, in
// lane l, D[4g + i][c] for i = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swimba {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef int int4v __attribute__((ext_vector_type(4)));

template <typename T> struct Vec;
template <> struct Vec<bf16> {
  typedef bf16x8 x8;
  typedef bf16x4 x4;
};
template <> struct Vec<f16> {
  typedef f16x8 x8;
  typedef f16x4 x4;
};
template <> struct Vec<float> {
  typedef floatx8 x8;
  typedef floatx4 x4;
};

// One K=32 step of a 16x16 tile: bf16 inputs, fp32 accumulation.
__device__ __forceinline__ floatx4 mma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mma16(f16x8 a, f16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The same contraction in fp32: eight 16x16x4 fp32 matrix-core ops. In op i,
// lane group g supplies element i of its fragment as contraction index g, so
// the eight ops together visit the same 32 (group, element) pairs.
__device__ __forceinline__ floatx4 mma16(floatx8 a, floatx8 b, floatx4 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }

// 16-byte global/LDS vector helpers.
template <typename T> __device__ __forceinline__ typename Vec<T>::x8 load8(const T* p);
template <> __device__ __forceinline__ bf16x8 load8<bf16>(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <> __device__ __forceinline__ f16x8 load8<f16>(const f16* p) {
  return *reinterpret_cast<const f16x8*>(p);
}
template <> __device__ __forceinline__ floatx8 load8<float>(const float* p) {
  floatx4 lo = *reinterpret_cast<const floatx4*>(p);
  floatx4 hi = *reinterpret_cast<const floatx4*>(p + 4);
  floatx8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

template <typename T> __device__ __forceinline__ void store8(T* p, typename Vec<T>::x8 v);
template <> __device__ __forceinline__ void store8<bf16>(bf16* p, bf16x8 v) {
  *reinterpret_cast<bf16x8*>(p) = v;
}
template <> __device__ __forceinline__ void store8<f16>(f16* p, f16x8 v) {
  *reinterpret_cast<f16x8*>(p) = v;
}
template <> __device__ __forceinline__ void store8<float>(float* p, floatx8 v) {
  floatx4 lo = {v[0], v[1], v[2], v[3]};
  floatx4 hi = {v[4], v[5], v[6], v[7]};
  *reinterpret_cast<floatx4*>(p) = lo;
  *reinterpret_cast<floatx4*>(p + 4) = hi;
}

template <typename T> __device__ __forceinline__ typename Vec<T>::x8 zero8() {
  typename Vec<T>::x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = from_f32<T>(0.f);
  return z;
}

// Two 4-element halves read from separate addresses, joined into a fragment.
template <typename T>
__device__ __forceinline__ typename Vec<T>::x8 load4x2(const T* p0, const T* p1) {
  typedef typename Vec<T>::x4 V4;
  V4 lo = *reinterpret_cast<const V4*>(p0);
  V4 hi = *reinterpret_cast<const V4*>(p1);
  typename Vec<T>::x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = lo[i];
    r[4 + i] = hi[i];
  }
  return r;
}

// Element type of the intermediate streams (B_hat, X_hat, C_mix) and of every
// matrix-core operand inside the scan, per input type: bf16 inputs keep their
// streams in fp16 (same bytes, 8x finer spacing; range +-65504), fp32 stays fp32.
template <typename TI> struct StreamOf;
template <> struct StreamOf<bf16> { typedef f16 type; };
template <> struct StreamOf<float> { typedef float type; };

// Convert 8 values between element types.
template <typename TO, typename TI>
__device__ __forceinline__ typename Vec<TO>::x8 convert8(typename Vec<TI>::x8 v) {
  typename Vec<TO>::x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = from_f32<TO>(to_f32(v[i]));
  return r;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Raw buffer resources: loads at a byte offset at or beyond the resource's
// size return zeros, so bounds handling is a select of the offset, not a
// branch. kOOB is an offset that is always out of range.
constexpr uint32_t kOOB = 0x80000000u;
typedef __amdgpu_buffer_rsrc_t BufRes;

__device__ __forceinline__ BufRes make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes >= 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// 8 elements (16 bytes for 2-byte types, 32 for fp32) at byte offset `off`.
template <typename T>
__device__ __forceinline__ typename Vec<T>::x8 load8_buf(BufRes r, uint32_t off) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(typename Vec<T>::x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  } else {
    int4v lo = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    int4v hi = __builtin_amdgcn_raw_buffer_load_b128(r, off >= kOOB ? kOOB : off + 16u, 0, 0);
    floatx4 a = __builtin_bit_cast(floatx4, lo), b = __builtin_bit_cast(floatx4, hi);
    floatx8 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
    return v;
  }
}

// a^n for a in [0, 1) and integer n >= 0, computed as exp2(n * log2(a)).
// a == 0 gives 1 for n == 0 and 0 otherwise.
__device__ __forceinline__ float pow_int(float a, int n) {
  if (n == 0) return 1.f;
  if (a <= 0.f) return 0.f;
  return exp2f((float)n * log2f(a));
}

}  // namespace swimba
