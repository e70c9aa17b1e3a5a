// Sampling verify after the logit rows have been streamed:
//  - k_sample_decide: one wave64 per request.  Lane i combines the split
//    partials of target row i and draft row i, evaluates p'(x_i), q'(x_i) in
//    fp64 and the test u_i * q'(x_i) < p'(x_i); a ballot over the lanes gives
//    the first rejection n (ariser.io review, section "같은 분포를 지키는 작은
//    장치": accept with probability min(1, p/q); lotook.com explainer, four
//    steps: scan left to right, stop at the first mismatch).
//  - k_resid_partial: per (split, request), the mass of max(0, p'_n - q'_n)
//    (or p'_K when every draft was accepted: the bonus token) over the split.
//  - k_sample_locate: per request, the inverse-CDF draw u * S over ascending
//    token ids: find the split, then the token inside it.
#include "sv_device.hpp"
#include "sv_kernels.hpp"

#pragma clang fp contract(off)

namespace sv {

namespace {

struct RowStatL {
  float m, tau;
  double z, zk;
};

__device__ RowStatL combine_row(const float *part_m, const double *part_z,
                                const RowStat *rowstat, int row, int S, double k64) {
  RowStatL r;
  if (rowstat) {
    const RowStat rs = rowstat[row];
    r.m = rs.m;
    r.tau = rs.tau;
    r.z = rs.z;
    r.zk = rs.zk;
    return r;
  }
  const float *pm = part_m + (size_t)row * S;
  const double *pz = part_z + (size_t)row * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, pm[s]);
  double Z = 0.0;
  for (int s = 0; s < S; ++s)
    if (pm[s] > -INFINITY) Z += pz[s] * exp2(((double)pm[s] - (double)M) * k64);
  r.m = M;
  r.tau = -INFINITY;
  r.z = Z;
  r.zk = Z;
  return r;
}

// p'(x) of one row at logit l (fp64): zero outside the nucleus.
__device__ __forceinline__ double prob_at(float l, const RowStatL &st, double k64) {
  if (!(l >= st.tau)) return 0.0;
  return exp2(((double)l - (double)st.m) * k64) / st.zk;
}

// Residual (or bonus) mass of one token; also its p' for the fallback.
// Both kernels that scan a row call this, so their per-token values agree.
__device__ __forceinline__ void resid_terms(float lt, float ld, const Decision &d, Scale k,
                                            double &r, double &p) {
  double pt = 0.0;
  if (lt >= d.tau_t) pt = (double)tempered(lt, d.m_t, k) * d.inv_t;
  p = pt;
  if (d.mode == kModeResidual) {
    double qd = 0.0;
    if (ld >= d.tau_d) qd = (double)tempered(ld, d.m_d, k) * d.inv_d;
    const double diff = pt - qd;
    r = diff > 0.0 ? diff : 0.0;
  } else {
    r = pt;
  }
}

__device__ __forceinline__ const char *row_ptr(const void *base, size_t row, int V, int dtype) {
  return (const char *)base + row * (size_t)V * elem_bytes(dtype);
}

}  // namespace

__global__ __launch_bounds__(64) void k_sample_decide(
    const char *__restrict__ target, const char *__restrict__ draft, int dtype,
    const int32_t *__restrict__ tokens, const float *__restrict__ u_accept, int B, int K,
    int V, int S, double k64, const float *__restrict__ part_m,
    const double *__restrict__ part_z, const RowStat *__restrict__ rowstat,
    int32_t *__restrict__ out_accepted, int32_t *__restrict__ out_tokens,
    float *__restrict__ out_p, float *__restrict__ out_q, Decision *__restrict__ dec) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int rows_t = B * (K + 1);
  RowStatL st_t{0.f, 0.f, 1.0, 1.0}, st_d{0.f, 0.f, 1.0, 1.0};
  if (i <= K) st_t = combine_row(part_m, part_z, rowstat, b * (K + 1) + i, S, k64);
  if (i < K) st_d = combine_row(part_m, part_z, rowstat, rows_t + b * K + i, S, k64);

  bool accept = false;
  int x = -1;
  if (i < K) {
    x = tokens[(size_t)b * K + i];
    double p = 0.0, q = 0.0;
    if (x >= 0 && x < V) {
      const float lt = load_elem(row_ptr(target, (size_t)b * (K + 1) + i, V, dtype), x, dtype);
      const float ld = load_elem(row_ptr(draft, (size_t)b * K + i, V, dtype), x, dtype);
      p = prob_at(lt, st_t, k64);
      q = prob_at(ld, st_d, k64);
      const double u = (double)u_accept[(size_t)b * K + i];
      accept = u * q < p;
    }
    if (out_p) out_p[(size_t)b * K + i] = (float)p;
    if (out_q) out_q[(size_t)b * K + i] = (float)q;
  }
  const uint64_t acc = __ballot(accept);
  const uint64_t live = K >= 64 ? ~0ull : ((1ull << K) - 1ull);
  const uint64_t rej = ~acc & live;
  const int n = rej ? __builtin_ctzll(rej) : K;
  if (i <= K) out_tokens[(size_t)b * (K + 1) + i] = i < n ? x : -1;
  if (i == 0) out_accepted[b] = n;
  if (i == n) {
    Decision d;
    d.n = n;
    d.mode = n < K ? kModeResidual : kModeBonus;
    d.m_t = st_t.m;
    d.tau_t = st_t.tau;
    d.inv_t = 1.0 / st_t.zk;
    d.m_d = st_d.m;
    d.tau_d = st_d.tau;
    d.inv_d = n < K ? 1.0 / st_d.zk : 0.0;
    dec[b] = d;
  }
}

// Residual partial sums over one split of target row n (and draft row n).
__global__ __launch_bounds__(kThreads) void k_resid_partial(
    const char *__restrict__ target, const char *__restrict__ draft, int dtype, int B, int K,
    int V, int S, Scale k, const Decision *__restrict__ dec, ResidPart *__restrict__ rpart) {
  const int b = blockIdx.x / S;
  const int s = blockIdx.x - b * S;
  const int t = threadIdx.x;
  const Decision d = dec[b];
  const char *rt = row_ptr(target, (size_t)b * (K + 1) + d.n, V, dtype);
  const char *rd = d.mode == kModeResidual ? row_ptr(draft, (size_t)b * K + d.n, V, dtype) : rt;
  const int C = split_elems(dtype);
  const int e0 = s * C;
  const int e1 = min(V, e0 + C);
  const int epv = 16 / elem_bytes(dtype);
  double sr = 0.0, spp = 0.0;
  int lr = -1, lp = -1;
  const Span st = split_span(rt, V, s, dtype);
  const Span sd = split_span(rd, V, s, dtype);
  if (st.head == sd.head) {
    // both rows share the 16-byte phase: vector body plus scalar head/tail
    const u32x4 *bt = span_body(st, dtype);
    const u32x4 *bd = span_body(sd, dtype);
    for (int v = t; v < st.nvec; v += kThreads) {
      const u32x4 wt = bt[v];
      const u32x4 wd = bd[v];
      const int j0 = e0 + st.head + v * epv;
      for (int e = 0; e < epv; ++e) {
        double r, p;
        resid_terms(vec_elem(wt, e, dtype), vec_elem(wd, e, dtype), d, k, r, p);
        sr += r;
        spp += p;
        if (r > 0.0) lr = j0 + e;
        if (p > 0.0) lp = j0 + e;
      }
    }
    const int se = span_scalar_elem(st, t, dtype);
    if (se >= 0) {
      double r, p;
      resid_terms(load_elem(rt, e0 + se, dtype), load_elem(rd, e0 + se, dtype), d, k, r, p);
      sr += r;
      spp += p;
      if (r > 0.0) lr = max(lr, e0 + se);
      if (p > 0.0) lp = max(lp, e0 + se);
    }
  } else {
    for (int j = e0 + t; j < e1; j += kThreads) {
      double r, p;
      resid_terms(load_elem(rt, j, dtype), load_elem(rd, j, dtype), d, k, r, p);
      sr += r;
      spp += p;
      if (r > 0.0) lr = j;
      if (p > 0.0) lp = j;
    }
  }
  // workgroup reduction
  __shared__ double s_r[kThreads / 64], s_p[kThreads / 64];
  __shared__ int s_lr[kThreads / 64], s_lp[kThreads / 64];
  sr = wave_sum(sr);
  spp = wave_sum(spp);
  for (int o = 32; o > 0; o >>= 1) {
    lr = max(lr, __shfl_xor(lr, o, 64));
    lp = max(lp, __shfl_xor(lp, o, 64));
  }
  if (lane_id() == 0) {
    s_r[t >> 6] = sr;
    s_p[t >> 6] = spp;
    s_lr[t >> 6] = lr;
    s_lp[t >> 6] = lp;
  }
  __syncthreads();
  if (t == 0) {
    ResidPart out;
    out.r = 0.0;
    out.p = 0.0;
    out.last_r = -1;
    out.last_p = -1;
    for (int w = 0; w < kThreads / 64; ++w) {
      out.r += s_r[w];
      out.p += s_p[w];
      out.last_r = max(out.last_r, s_lr[w]);
      out.last_p = max(out.last_p, s_lp[w]);
    }
    rpart[(size_t)b * S + s] = out;
  }
}

// Inverse CDF over ascending ids: the smallest j with C_j > u * S.
__global__ __launch_bounds__(kThreads) void k_sample_locate(
    const char *__restrict__ target, const char *__restrict__ draft, int dtype,
    const float *__restrict__ u_sample, int B, int K, int V, int S, Scale k,
    const Decision *__restrict__ dec, const ResidPart *__restrict__ rpart,
    int32_t *__restrict__ out_tokens, float *__restrict__ out_mass) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const Decision d = dec[b];
  const ResidPart *rp = rpart + (size_t)b * S;
  __shared__ int s_split, s_use_p, s_token;
  __shared__ double s_rem, s_total;
  if (t == 0) {
    double Sr = 0.0;
    for (int s = 0; s < S; ++s) Sr += rp[s].r;
    int use_p = 0;
    double tot = Sr;
    if (!(Sr > 0.0)) {  // unreachable in exact arithmetic after a rejection
      use_p = 1;
      tot = 0.0;
      for (int s = 0; s < S; ++s) tot += rp[s].p;
    }
    const double target_mass = (double)u_sample[b] * tot;
    double c = 0.0;
    int split = -1;
    for (int s = 0; s < S; ++s) {
      const double v = use_p ? rp[s].p : rp[s].r;
      if (c + v > target_mass) {
        split = s;
        break;
      }
      c += v;
    }
    int token = -1;
    if (split < 0) {  // rounding left no crossing: the last token with mass
      for (int s = S - 1; s >= 0 && token < 0; --s) token = use_p ? rp[s].last_p : rp[s].last_r;
    }
    s_split = split;
    s_use_p = use_p;
    s_token = token;
    s_rem = target_mass - c;
    s_total = tot;
  }
  __syncthreads();
  const int split = s_split;
  if (split >= 0) {
    const int use_p = s_use_p;
    const double rem = s_rem;
    const char *rt = row_ptr(target, (size_t)b * (K + 1) + d.n, V, dtype);
    const char *rd = d.mode == kModeResidual ? row_ptr(draft, (size_t)b * K + d.n, V, dtype) : rt;
    const int C = split_elems(dtype);
    const int e0 = split * C;
    const int e1 = min(V, e0 + C);
    const int per = (e1 - e0 + kThreads - 1) / kThreads;
    const int j0 = e0 + t * per;
    const int j1 = min(e1, j0 + per);
    double own = 0.0;
    for (int j = j0; j < j1; ++j) {
      double r, p;
      resid_terms(load_elem(rt, j, dtype), load_elem(rd, j, dtype), d, k, r, p);
      own += use_p ? p : r;
    }
    // exclusive scan of the per-thread sums (ascending thread = ascending ids)
    __shared__ double scan[kThreads];
    scan[t] = own;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const double v = t >= off ? scan[t - off] : 0.0;
      __syncthreads();
      scan[t] += v;
      __syncthreads();
    }
    // [scan[t-1], scan[t]) partition [0, scan[last]): at most one thread
    // holds the crossing and walks its range element by element
    const double before = t > 0 ? scan[t - 1] : 0.0;
    if (before <= rem && rem < scan[t] && j0 < j1) {
      double c = before;
      int pick = -1, last_pos = -1;
      for (int j = j0; j < j1; ++j) {
        double r, p;
        resid_terms(load_elem(rt, j, dtype), load_elem(rd, j, dtype), d, k, r, p);
        const double v = use_p ? p : r;
        if (v > 0.0) last_pos = j;
        c += v;
        if (c > rem) {
          pick = j;
          break;
        }
      }
      s_token = pick >= 0 ? pick : last_pos;
    }
    __syncthreads();
    if (t == 0 && s_token < 0) s_token = use_p ? rp[split].last_p : rp[split].last_r;
    __syncthreads();
  }
  if (t == 0) {
    out_tokens[(size_t)b * (K + 1) + d.n] = s_token;
    if (out_mass) out_mass[b] = (float)s_total;
  }
}

hipError_t launch_sample_decide(const void *target, const void *draft, int dtype,
                                const int32_t *tokens, const float *u_accept, int B, int K,
                                int V, int S, double k64, const float *part_m,
                                const double *part_z, const RowStat *rowstat,
                                int32_t *out_accepted, int32_t *out_tokens, float *out_p,
                                float *out_q, Decision *dec, hipStream_t stream) {
  hipLaunchKernelGGL(k_sample_decide, dim3(B), dim3(64), 0, stream, (const char *)target,
                     (const char *)draft, dtype, tokens, u_accept, B, K, V, S, k64, part_m,
                     part_z, rowstat, out_accepted, out_tokens, out_p, out_q, dec);
  return hipGetLastError();
}

hipError_t launch_resid_partial(const void *target, const void *draft, int dtype, int B,
                                int K, int V, int S, Scale k, const Decision *dec,
                                ResidPart *rpart, hipStream_t stream) {
  hipLaunchKernelGGL(k_resid_partial, dim3(S * B), dim3(kThreads), 0, stream,
                     (const char *)target, (const char *)draft, dtype, B, K, V, S, k, dec,
                     rpart);
  return hipGetLastError();
}

hipError_t launch_sample_locate(const void *target, const void *draft, int dtype,
                                const float *u_sample, int B, int K, int V, int S, Scale k,
                                const Decision *dec, const ResidPart *rpart,
                                int32_t *out_tokens, float *out_mass, hipStream_t stream) {
  hipLaunchKernelGGL(k_sample_locate, dim3(B), dim3(kThreads), 0, stream,
                     (const char *)target, (const char *)draft, dtype, u_sample, B, K, V, S,
                     k, dec, rpart, out_tokens, out_mass);
  return hipGetLastError();
}

}  // namespace sv
