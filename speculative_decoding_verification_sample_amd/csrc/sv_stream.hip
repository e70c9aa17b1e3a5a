// Logit streaming kernels: every logit row is read from HBM exactly once,
// one workgroup per (split, row), 256 lanes x 8 16-byte loads in flight.
//
//  - k_softmax_partial: per split, the maximum m and the tempered mass
//    z = sum 2^((l - m) k) (the softmax normaliser at temperature T, with
//    k = log2(e)/T), fp32 terms accumulated in fp64.  Temperature is applied
//    to target and draft rows alike (ariser.io review, section
//    "같은 분포를 지키는 작은 장치": p and q must reflect the sampling settings).
//  - k_argmax_partial: per split, the largest value and its lowest index,
//    packed into one 64-bit key so that max() resolves ties to the lowest id
//    (greedy verification compares drafts with the target's top choice:
//    lotook.com explainer, four steps / FAQ).
#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {

template <int DT>
__device__ __forceinline__ u32x4 neg_inf_vec() {
  const uint32_t w = DT == kBF16 ? 0xFF80FF80u : 0xFF800000u;
  u32x4 v = {w, w, w, w};
  return v;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_softmax_partial(
    const char *__restrict__ target, const char *__restrict__ draft, int rows_t, int V,
    int S, Scale k, float *__restrict__ part_m, double *__restrict__ part_z) {
  constexpr int EPV = 16 / elem_bytes(DT);
  const int row = blockIdx.x / S;
  const int s = blockIdx.x - row * S;
  const size_t row_bytes = (size_t)V * elem_bytes(DT);
  const char *rp = row < rows_t ? target + (size_t)row * row_bytes
                                : draft + (size_t)(row - rows_t) * row_bytes;
  const Span sp = split_span(rp, V, s, DT);
  const u32x4 *body = span_body(sp, DT);
  const int t = threadIdx.x;

  u32x4 buf[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const int v = t + u * kThreads;
    buf[u] = v < sp.nvec ? body[v] : neg_inf_vec<DT>();
  }
  const int se = span_scalar_elem(sp, t, DT);
  const float xs = se >= 0 ? load_elem(sp.base, se, DT) : -INFINITY;

  float m = xs;
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u)
#pragma unroll
    for (int e = 0; e < EPV; ++e) m = fmaxf(m, vec_elem(buf[u], e, DT));

  double z = 0.0;
  if (m > -INFINITY) {
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int e = 0; e < EPV; e += 2) {
        a0 += tempered(vec_elem(buf[u], e, DT), m, k);
        a1 += tempered(vec_elem(buf[u], e + 1, DT), m, k);
      }
      z += (double)(a0 + a1);
    }
    if (se >= 0) z += (double)tempered(xs, m, k);
  }

  // workgroup combine: rescale each lane's sum to the wave maximum, then to
  // the workgroup maximum (factors <= 1, computed from exact differences)
  __shared__ float sm[kThreads / 64];
  __shared__ double sz[kThreads / 64];
  const float wm = wave_max(m);
  double zz = (m > -INFINITY) ? z * (double)tempered(m, wm, k) : 0.0;
  zz = wave_sum(zz);
  if (lane_id() == 0) {
    sm[t >> 6] = wm;
    sz[t >> 6] = zz;
  }
  __syncthreads();
  if (t == 0) {
    float M = sm[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, sm[w]);
    double Z = 0.0;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w)
        if (sm[w] > -INFINITY) Z += sz[w] * (double)tempered(sm[w], M, k);
    }
    const size_t cell = (size_t)row * S + s;
    part_m[cell] = M;
    part_z[cell] = Z;
  }
}

// 64-bit argmax key: order-preserving value key in the high word, the
// complement of the element index in the low word (ties -> lowest index).
__device__ __forceinline__ uint64_t argmax_key(float x, uint32_t idx) {
  return ((uint64_t)key_of_f32(x) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_argmax_partial(
    const char *__restrict__ logits, int V, int S, uint64_t *__restrict__ part_key) {
  constexpr int EPV = 16 / elem_bytes(DT);
  const int row = blockIdx.x / S;
  const int s = blockIdx.x - row * S;
  const size_t row_bytes = (size_t)V * elem_bytes(DT);
  const Span sp = split_span(logits + (size_t)row * row_bytes, V, s, DT);
  const u32x4 *body = span_body(sp, DT);
  const int t = threadIdx.x;

  u32x4 buf[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const int v = t + u * kThreads;
    buf[u] = v < sp.nvec ? body[v] : neg_inf_vec<DT>();
  }
  uint64_t best = 0;
  const int se = span_scalar_elem(sp, t, DT);
  if (se >= 0) best = argmax_key(load_elem(sp.base, se, DT), (uint32_t)(sp.e0 + se));
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const int v = t + u * kThreads;
    if (v < sp.nvec) {
      const uint32_t i0 = (uint32_t)(sp.e0 + sp.head + v * EPV);
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const uint64_t key = argmax_key(vec_elem(buf[u], e, DT), i0 + e);
        best = key > best ? key : best;
      }
    }
  }
  __shared__ uint64_t sk[kThreads / 64];
  best = wave_max_u64(best);
  if (lane_id() == 0) sk[t >> 6] = best;
  __syncthreads();
  if (t == 0) {
    uint64_t b = sk[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) b = sk[w] > b ? sk[w] : b;
    part_key[(size_t)row * S + s] = b;
  }
}

hipError_t launch_softmax_partial(const void *target, const void *draft, int dtype,
                                  int rows_t, int rows_d, int V, int S, Scale k,
                                  float *part_m, double *part_z, hipStream_t stream) {
  dim3 grid(S * (rows_t + rows_d)), block(kThreads);
  if (dtype == kBF16)
    hipLaunchKernelGGL(k_softmax_partial<kBF16>, grid, block, 0, stream,
                       (const char *)target, (const char *)draft, rows_t, V, S, k, part_m,
                       part_z);
  else
    hipLaunchKernelGGL(k_softmax_partial<kF32>, grid, block, 0, stream,
                       (const char *)target, (const char *)draft, rows_t, V, S, k, part_m,
                       part_z);
  return hipGetLastError();
}

hipError_t launch_argmax_partial(const void *logits, int dtype, int rows, int V, int S,
                                 uint64_t *part_key, hipStream_t stream) {
  dim3 grid(S * rows), block(kThreads);
  if (dtype == kBF16)
    hipLaunchKernelGGL(k_argmax_partial<kBF16>, grid, block, 0, stream,
                       (const char *)logits, V, S, part_key);
  else
    hipLaunchKernelGGL(k_argmax_partial<kF32>, grid, block, 0, stream,
                       (const char *)logits, V, S, part_key);
  return hipGetLastError();
}

}  // namespace sv
