// Device helpers for the gfx950 verify kernels: logit row geometry, 16-byte
// vector loads, bf16 widening, order-preserving keys, wave64 reductions and
// the split exponent used for tempered softmax masses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_layout.hpp"

namespace sv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// row / split geometry
// ---------------------------------------------------------------------------

// The elements [e0, e0 + n) of one split, cut into a scalar head (until the
// first 16-byte boundary), a body of 16-byte vectors and a scalar tail.
struct Span {
  const char *base;  // address of element e0
  int e0;            // first element (row-relative)
  int n;             // elements in the split
  int head;          // scalar elements before the body
  int nvec;          // 16-byte vectors in the body
  int tail;          // scalar elements after the body
};

__device__ __forceinline__ Span split_span(const char *row, int V, int s, int dtype) {
  const int es = elem_bytes(dtype);
  const int epv = 16 / es;
  Span sp;
  sp.e0 = s * split_elems(dtype);
  int e1 = min(V, sp.e0 + split_elems(dtype));
  sp.n = max(0, e1 - sp.e0);
  sp.base = row + (size_t)sp.e0 * es;
  uintptr_t a = reinterpret_cast<uintptr_t>(sp.base);
  int head = (int)(((16u - (unsigned)(a & 15u)) & 15u) / (unsigned)es);
  sp.head = min(head, sp.n);
  int rest = sp.n - sp.head;
  sp.nvec = rest / epv;
  sp.tail = rest - sp.nvec * epv;
  return sp;
}

// Scalar element handled by thread t (head first, then tail); -1 if none.
__device__ __forceinline__ int span_scalar_elem(const Span &sp, int t, int dtype) {
  if (t < sp.head) return t;
  int u = t - sp.head;
  if (u < sp.tail) return sp.head + sp.nvec * (16 / elem_bytes(dtype)) + u;
  return -1;
}

__device__ __forceinline__ const u32x4 *span_body(const Span &sp, int dtype) {
  return reinterpret_cast<const u32x4 *>(sp.base + (size_t)sp.head * elem_bytes(dtype));
}

// ---------------------------------------------------------------------------
// element access
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Element i of a logit row, widened exactly to fp32.
__device__ __forceinline__ float load_elem(const char *row, size_t i, int dtype) {
  if (dtype == kBF16) {
    uint32_t h = reinterpret_cast<const uint16_t *>(row)[i];
    return __uint_as_float(h << 16);
  }
  return reinterpret_cast<const float *>(row)[i];
}

// Element k (0..epv-1) of a 16-byte vector.
__device__ __forceinline__ float vec_elem(const u32x4 &v, int k, int dtype) {
  if (dtype == kBF16) {
    uint32_t w = v[k >> 1];
    return (k & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  return __uint_as_float(v[k]);
}

// ---------------------------------------------------------------------------
// order-preserving keys: larger value <-> larger key, -0.0 and +0.0 equal
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t key_of_f32(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t mag = u & 0x7FFFFFFFu;
  return (u >> 31) ? 0x80000000u - mag : 0x80000000u + mag;
}

__device__ __forceinline__ float f32_of_key(uint32_t k) {
  return k >= 0x80000000u ? __uint_as_float(k - 0x80000000u)
                          : __uint_as_float((0x80000000u - k) | 0x80000000u);
}

// ---------------------------------------------------------------------------
// tempered masses: exp((l - m) / T) = 2^((l - m) * k), k = log2(e) / T held as
// k_hi + k_lo so that the product carries ~1 ulp of error per element rather
// than the rounding of k itself (which would act like a shifted temperature).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float exp2_fast(float a) { return __builtin_amdgcn_exp2f(a); }

__device__ __forceinline__ float tempered(float l, float m, Scale k) {
  float d = l - m;
  return exp2_fast(fmaf(d, k.hi, d * k.lo));
}

// ---------------------------------------------------------------------------
// wave64 reductions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

}  // namespace sv
