// Streaming tiles: one split of one logit row per 256-lane workgroup, every
// lane with 8 nontemporal 16-byte loads in flight.  Called by the whole
// workgroup; the result is valid in thread 0.
#pragma once

#include "sv_device.hpp"

namespace sv {

template <int DT>
__device__ __forceinline__ u32x4 neg_inf_vec() {
  const uint32_t w = DT == kBF16 ? 0xFF80FF80u : 0xFF800000u;
  u32x4 v = {w, w, w, w};
  return v;
}

// Softmax statistics of split s of row `rp`: the maximum M and the tempered
// mass Z = sum 2^((l - M) k), fp32 terms accumulated in fp64.  `pre` runs
// once the tile's loads are in flight (work that must not delay them).  With
// `hist`, the split's elements are also counted by bin j = floor(M kk) -
// floor(l kk), kk = k * kHistPerLog2 (bins of 1/64 log2 unit on a grid shared
// by all splits, so that counts merge across splits by integer offsets);
// bins past kHistBins are not counted.  With `hist`, `cmax` takes the
// split's chunk maxima (kChunksPerSplit entries, fp32 patterns) and `cmax2`
// a bound on each chunk's second largest element (f32_hi_up of it).  HIST
// false compiles none of it (the pointers are then ignored).
template <int DT, bool HIST, class Pre>
__device__ __forceinline__ void softmax_tile(const char *rp, int V, int s, Scale k, float *M_out,
                                             double *Z_out, Pre &&pre, uint8_t *hist,
                                             uint32_t *cmax, uint16_t *cmax2) {
  constexpr int EPV = 16 / elem_bytes(DT);
  const Span sp = split_span(rp, V, s, DT);
  const u32x4 *body = span_body(sp, DT);
  const int t = threadIdx.x;
  __shared__ unsigned sh_hist[kHistBins + 64];  // + one spare slot per lane (not written out)
  if (hist)
    for (int i = t; i < kHistBins; i += kThreads) sh_hist[i] = 0u;

  u32x4 buf[kVecPerThread];
  if (sp.nvec == kThreads * kVecPerThread) {  // a whole split (all but a row's last): no checks
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) buf[u] = load_stream(body + t + u * kThreads);
  } else {
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const int v = t + u * kThreads;
      buf[u] = v < sp.nvec ? load_stream(body + v) : neg_inf_vec<DT>();
    }
  }
  const int se = span_scalar_elem(sp, t, DT);
  const float xs = se >= 0 ? load_elem(sp.base, se, DT) : -INFINITY;
  pre();

  // HIST: each slot's largest and second largest element over the lane's
  // elements (the second by a median of three: med3(first, second, x) is
  // the new second whenever first >= second).  fp32 slots (four elements)
  // take them here, in place of the plain maximum; bf16 slots (eight, each
  // widened here and again below) take them in the exponential pass, where
  // each widened element is at hand (here they would keep all 64 widened
  // elements live: 149 registers instead of 93).
  constexpr bool kTop2First = DT == kF32;
  float m = xs;
  float mu[kVecPerThread], mv[kVecPerThread];
  if constexpr (HIST && kTop2First) {
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      mu[u] = vec_elem(buf[u], 0, DT);
      mv[u] = -INFINITY;
#pragma unroll
      for (int e = 1; e < EPV; ++e) {
        const float x = vec_elem(buf[u], e, DT);
        mv[u] = __builtin_amdgcn_fmed3f(mu[u], mv[u], x);
        mu[u] = fmaxf(mu[u], x);
      }
      m = fmaxf(m, mu[u]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u)
#pragma unroll
      for (int e = 0; e < EPV; ++e) m = fmaxf(m, vec_elem(buf[u], e, DT));
    if constexpr (HIST) {
#pragma unroll
      for (int u = 0; u < kVecPerThread; ++u) mu[u] = mv[u] = -INFINITY;
    }
  }

  // 2^((l - m) k) with k = hi + lo: the exponent is taken as
  // (l hi + c) + l lo with c = -m hi rounded to a float (two fused
  // multiply-adds, each product exact); the parts left out, the rounding
  // e = -m hi - c (exact by one more fused multiply-add) and -m lo, are
  // the same for every element and scale the lane's sum once, in fp64.
  double z = 0.0;
  if (m > -INFINITY) {
    const float c = -m * k.hi;
    const float e = fmaf(-m, k.hi, -c);
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      auto term = [&](int j) {
        const float x = vec_elem(buf[u], j, DT);
        return exp2_fast(fmaf(x, k.lo, fmaf(x, k.hi, c)));
      };
      float a0 = term(0), a1 = term(1);
#pragma unroll
      for (int j = 2; j < EPV; j += 2) {
        a0 += term(j);
        a1 += term(j + 1);
      }
      z += (double)(a0 + a1);
      if constexpr (HIST && !kTop2First) {
#pragma unroll
        for (int j = 0; j < EPV; ++j) {
          const float x = vec_elem(buf[u], j, DT);
          mv[u] = __builtin_amdgcn_fmed3f(mu[u], mv[u], x);
          mu[u] = fmaxf(mu[u], x);
        }
      }
    }
    if (se >= 0) z += (double)exp2_fast(fmaf(xs, k.lo, fmaf(xs, k.hi, c)));
    // 2^delta for |delta| < 1e-5: 1 + delta ln2 + (delta ln2)^2 / 2, error < 1e-16
    const double dl = ((double)e - (double)m * (double)k.lo) * 0.6931471805599453;
    z *= 1.0 + dl * (1.0 + 0.5 * dl);
  }

  // rescale each lane's sum to the wave maximum, then to the workgroup
  // maximum (factors <= 1, computed from exact differences)
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
  if (HIST && hist) {
    // chunk maxima and second elements: slot u's lane pairs (largest,
    // second), reduced over the group of eight lanes by a reduce-scatter of
    // three exchanges (partner 7 - i, i ^ 2, i ^ 1), each lane keeping the
    // half of its slots whose index bit matches its own lane bit and sending
    // the other half: lane t ends with slot t % 8's pair.  Two pairs merge
    // as (max of the firsts, max(min of the firsts, max of the seconds)).
    const uint32_t ninf = __float_as_uint(-INFINITY);
    const int li = t & (kChunkLanes - 1);
    auto merge = [](float &a1, float &a2, float b1, float b2) {
      a2 = fmaxf(fminf(a1, b1), fmaxf(a2, b2));
      a1 = fmaxf(a1, b1);
    };
    float p4[4], q4[4], p2[2], q2[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool hi = li & 4;
      p4[j] = hi ? mu[j + 4] : mu[j];
      q4[j] = hi ? mv[j + 4] : mv[j];
      const float s1 = hi ? mu[j] : mu[j + 4], s2 = hi ? mv[j] : mv[j + 4];
      merge(p4[j], q4[j], __uint_as_float(dpp_u32<kDppHalfMirror>(ninf, __float_as_uint(s1))),
            __uint_as_float(dpp_u32<kDppHalfMirror>(ninf, __float_as_uint(s2))));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool hi = li & 2;
      p2[j] = hi ? p4[j + 2] : p4[j];
      q2[j] = hi ? q4[j + 2] : q4[j];
      const float s1 = hi ? p4[j] : p4[j + 2], s2 = hi ? q4[j] : q4[j + 2];
      merge(p2[j], q2[j], __uint_as_float(dpp_u32<kDppXor2>(ninf, __float_as_uint(s1))),
            __uint_as_float(dpp_u32<kDppXor2>(ninf, __float_as_uint(s2))));
    }
    {
      const bool hi = li & 1;
      float p1 = hi ? p2[1] : p2[0], q1 = hi ? q2[1] : q2[0];
      const float s1 = hi ? p2[0] : p2[1], s2 = hi ? q2[0] : q2[1];
      merge(p1, q1, __uint_as_float(dpp_u32<kDppXor1>(ninf, __float_as_uint(s1))),
            __uint_as_float(dpp_u32<kDppXor1>(ninf, __float_as_uint(s2))));
      cmax[t] = __float_as_uint(p1);
      cmax2[t] = (uint16_t)f32_hi_up(q1);
    }
    float M = sm[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, sm[w]);
    if (M > -INFINITY) {
      const float kk = (k.hi + k.lo) * kHistPerLog2;
      // F = floor(M kk) as an integer: |M kk| < 2^31 wherever the counts are
      // used (the band launch requires |M kk| < 2^18)
      const unsigned F = (unsigned)floor_to_int(M * kk);
      // branch-free: j = F - floor(x kk) >= 0 (x <= M) in unsigned
      // arithmetic; -inf (INT_MIN) and everything past the counted bins give
      // j >= kHistBins, which the minimum sends to a spare slot beyond the
      // bins (the lane's own, or one of a lane below: never read back)
      const unsigned spare = kHistBins + lane_id();
      auto count = [&](float x) {
        const unsigned j = F - (unsigned)floor_to_int(x * kk);
        atomicAdd(&sh_hist[min(j, spare)], 1u);
      };
#pragma unroll
      for (int u = 0; u < kVecPerThread; ++u)
#pragma unroll
        for (int e = 0; e < EPV; ++e) count(vec_elem(buf[u], e, DT));
      if (se >= 0) count(xs);
    }
    __syncthreads();
    uint32_t *h4 = reinterpret_cast<uint32_t *>(hist);
    for (int i = t; i < kHistBins / 4; i += kThreads)
      h4[i] = min(sh_hist[4 * i], kCountSat) | (min(sh_hist[4 * i + 1], kCountSat) << 8) |
              (min(sh_hist[4 * i + 2], kCountSat) << 16) | (min(sh_hist[4 * i + 3], kCountSat) << 24);
  }
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
    *M_out = M;
    *Z_out = Z;
  }
}

// 64-bit argmax key: order-preserving value key in the high word, the
// complement of the element index in the low word (ties -> lowest index).
__device__ __forceinline__ uint64_t argmax_key(float x, uint32_t idx) {
  return ((uint64_t)key_of_f32(x) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

// The lane's best key over its part of the split (FULL: a whole split, no
// bounds checks).
template <int DT, bool FULL>
__device__ __forceinline__ uint64_t argmax_lane(const Span &sp, const u32x4 *body, int t) {
  constexpr int EPV = 16 / elem_bytes(DT);
  u32x4 buf[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const int v = t + u * kThreads;
    buf[u] = (FULL || v < sp.nvec) ? load_stream(body + v) : neg_inf_vec<DT>();
  }
  uint64_t best = 0;
  const int se = span_scalar_elem(sp, t, DT);
  if (se >= 0) best = argmax_key(load_elem(sp.base, se, DT), (uint32_t)(sp.e0 + se));
  // the lane's maximum, then the lowest index holding it (the lane's
  // elements ascend with u, then e): 1.5 + 2 operations per element instead
  // of a 64-bit key comparison each
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u)
#pragma unroll
    for (int e = 0; e < EPV; ++e) m = fmaxf(m, vec_elem(buf[u], e, DT));
  int first = -1;
#pragma unroll
  for (int u = kVecPerThread - 1; u >= 0; --u) {
    const int v = t + u * kThreads;
    if (FULL || v < sp.nvec) {
      const int i0 = sp.e0 + sp.head + v * EPV;
#pragma unroll
      for (int e = EPV - 1; e >= 0; --e) first = vec_elem(buf[u], e, DT) == m ? i0 + e : first;
    }
  }
  if (first >= 0) {
    const uint64_t key = argmax_key(m, (uint32_t)first);
    best = key > best ? key : best;
  }
  return best;
}

template <int DT>
__device__ __forceinline__ uint64_t argmax_tile(const char *rp, int V, int s) {
  const Span sp = split_span(rp, V, s, DT);
  const u32x4 *body = span_body(sp, DT);
  const int t = threadIdx.x;
  uint64_t best = sp.nvec == kThreads * kVecPerThread ? argmax_lane<DT, true>(sp, body, t)
                                                      : argmax_lane<DT, false>(sp, body, t);
  __shared__ uint64_t sk[kThreads / 64];
  best = wave_max_u64(best);
  if (lane_id() == 0) sk[t >> 6] = best;
  __syncthreads();
  uint64_t b = sk[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) b = sk[w] > b ? sk[w] : b;
  return b;
}

}  // namespace sv
