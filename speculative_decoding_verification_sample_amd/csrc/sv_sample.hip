// Sampling verify in one kernel, k_sample_fused.  Blocks come in groups
// g = 0 .. B+L-1: the streaming tiles of request g (one per row split), then
// the residual tiles of request g - L (one per residual split).  A residual
// tile is dispatched after every tile it waits for (its request's streaming
// tiles, L groups earlier, and its sibling residual tiles, adjacent to it),
// so it only ever waits for work that is already running (a bounded wait,
// never forever), while the residual work of early requests overlaps the
// streaming of later ones.  L is about one resident wave of requests.  Partials
// are self-validating words carrying the call's epoch bits, so the workspace
// needs no clearing between calls, a partial is published with one store and
// read (and validated) with one load, and no tile performs an atomic
// read-modify-write.
//
// Streaming tile: the split's (max, tempered mass) partial, two words.
// Residual tile (b, s), once request b's rows are all streamed:
//  1. decide: combine the (2K+1) x S partials, evaluate p'(x_i), q'(x_i) in
//     fp64 and the test u_i * q'(x_i) < p'(x_i); a ballot gives the first
//     rejection n (ariser.io review, section "같은 분포를 지키는 작은 장치":
//     accept with probability min(1, p/q); lotook.com explainer, four steps:
//     scan left to right, stop at the first mismatch).  Split 0 writes the
//     accepted drafts.
//  2. sum the residual mass max(0, p'_n - q'_n) over the split (p'_K when all
//     K drafts survived: the bonus token), fp32 terms into fp64, and publish.
//  3. the request's last residual tile (dispatched after its siblings)
//     gathers the split masses, finds the split where the cumulative mass
//     passes u * S (inverse CDF over ascending ids), reads that split again,
//     scans its per-group masses and one lane walks to the token.  The other
//     residual tiles exit after publishing.
// With top-p the same kernel runs twice (streaming tiles only, then residual
// tiles only) around the nucleus kernel, which fills RowStat.
#include <algorithm>

#include "sv_device.hpp"
#include "sv_kernels.hpp"
#include "sv_tiles.hpp"

#pragma clang fp contract(off)

namespace sv {

namespace {

constexpr int kMaxCells = 1024;  // (2K+1) x S partials combined in LDS
constexpr int kEntries = kThreads * kVecPerThreadB + 2;
constexpr int kNoEntry = 0x7FFFFFFF;

// LDS shared by the decide and draw phases of a residual tile.
struct DecideLds {
  float cell_m[kMaxCells];
  double cell_z[kMaxCells];
  float row_m[128], row_tau[128];
  double row_zk[128];
};
struct DrawLds {
  double pr[kMaxSplitsB], pp[kMaxSplitsB];
  int plr[kMaxSplitsB], plp[kMaxSplitsB];
  double val[kEntries];
  double tsum[kThreads];
};
union TileLds {
  DecideLds dec;
  DrawLds draw;
};

// p'(x) of one row at logit l (fp64): zero outside the nucleus.
__device__ __forceinline__ double prob_at(float l, float m, float tau, double zk, double k64) {
  if (!(l >= tau)) return 0.0;
  return exp2(((double)l - (double)m) * k64) / zk;
}

// Residual (or bonus) mass of one token, and its p' for the fallback.  Every
// pass that scans a row calls this, so the per-token values agree bit for bit.
// Branch-free: for the bonus draw the draft weight inv_d is 0 (and m_d, tau_d
// repeat the target's), so r = max(p' - 0, 0) = p'.
__device__ __forceinline__ void resid_terms(float lt, float ld, const Decision &d, Scale k,
                                            double &r, double &p) {
  const double et = (double)tempered(lt, d.m_t, k) * d.inv_t;
  const double eq = (double)tempered(ld, d.m_d, k) * d.inv_d;
  const double pt = lt >= d.tau_t ? et : 0.0;
  const double qd = ld >= d.tau_d ? eq : 0.0;
  const double diff = pt - qd;
  r = diff > 0.0 ? diff : 0.0;
  p = pt;
}

__device__ __forceinline__ const char *row_ptr(const void *base, size_t row, int V, int dtype) {
  return (const char *)base + row * (size_t)V * elem_bytes(dtype);
}

// One 16-byte group of elements starting at p; assembled from scalar loads
// when p is not 16-byte aligned.
template <int DT>
__device__ __forceinline__ u32x4 load_group(const char *p, bool aligned) {
  if (aligned) return *reinterpret_cast<const u32x4 *>(p);
  u32x4 r;
  if (DT == kBF16) {
    const uint16_t *h = reinterpret_cast<const uint16_t *>(p);
#pragma unroll
    for (int w = 0; w < 4; ++w) r[w] = (uint32_t)h[2 * w] | ((uint32_t)h[2 * w + 1] << 16);
  } else {
    const uint32_t *f = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
    for (int w = 0; w < 4; ++w) r[w] = f[w];
  }
  return r;
}

// Poll one (row, split) cell until it carries this call's epoch.
__device__ __forceinline__ bool read_cell(const u64 *part_m, const u64 *part_z, size_t g,
                                          u64 epoch, float *m, double *z) {
  for (int it = 0; it < kSpinLimit; ++it) {
    const u64 mw = load_agent(&part_m[g]);
    const u64 zw = load_agent(&part_z[g]);
    if (unpack_f32(mw, epoch, m) & unpack_f64(zw, epoch, z)) return true;
    spin_pause();
  }
  return false;
}

// The accept / reject outcome of request b into *sd; whole workgroup.
// Returns false if a partial never arrived (bounded wait timed out).
__device__ bool decide(const int32_t *tokens, const float *u_accept, int B, int K, int S,
                       double k64, const u64 *part_m, const u64 *part_z, const u64 *part_x,
                       u64 epoch,
                       const RowStat *rowstat, int b, bool write_outputs, int32_t *out_accepted,
                       int32_t *out_tokens, float *out_p, float *out_q, DecideLds &L,
                       Decision *sd, int *flag) {
  const int t = threadIdx.x;
  const int R = 2 * K + 1;  // local rows: target 0..K, draft K+1..2K
  const int rows_t = B * (K + 1);
  auto global_row = [&](int r) {
    return r <= K ? b * (K + 1) + r : rows_t + b * K + (r - K - 1);
  };
  if (t == 0) *flag = 1;
  // the draft tokens (for the emitted prefix) and their logits (lanes < K):
  // the logits come from the streaming tiles, -inf for a token out of range
  int x = -1;
  float lt = -INFINITY, ld = -INFINITY;
  bool got_x = true;
  if (t < K) {
    x = tokens[(size_t)b * K + t];
    const u64 *px = part_x + ((size_t)b * K + t) * 2;
    got_x = false;
    for (int it = 0; it < kSpinLimit && !got_x; ++it) {
      uint32_t bt, bd;
      got_x = unpack_u32(load_agent(&px[0]), epoch, &bt) & unpack_u32(load_agent(&px[1]), epoch, &bd);
      lt = __uint_as_float(bt);
      ld = __uint_as_float(bd);
      if (!got_x) spin_pause();
    }
  }
  __syncthreads();
  if (!got_x) *flag = 0;
  if (rowstat) {
    if (t < R) {
      const RowStat rs = rowstat[global_row(t)];
      L.row_m[t] = rs.m;
      L.row_tau[t] = rs.tau;
      L.row_zk[t] = rs.zk;
    }
  } else if (R * S <= kMaxCells) {
    bool ok = true;
    for (int c = t; c < R * S; c += kThreads) {
      float m = -INFINITY;
      double z = 0.0;
      ok = ok && read_cell(part_m, part_z, (size_t)global_row(c / S) * S + (c % S), epoch, &m, &z);
      L.cell_m[c] = m;
      L.cell_z[c] = z;
    }
    if (!ok) *flag = 0;
    __syncthreads();
    if (t < R) {
      float M = -INFINITY;
      for (int s2 = 0; s2 < S; ++s2) M = fmaxf(M, L.cell_m[t * S + s2]);
      L.row_m[t] = M;
      L.row_tau[t] = -INFINITY;
    }
    __syncthreads();
    for (int c = t; c < R * S; c += kThreads) {
      const float m = L.cell_m[c], M = L.row_m[c / S];
      L.cell_z[c] = m > -INFINITY ? L.cell_z[c] * exp2(((double)m - (double)M) * k64) : 0.0;
    }
    __syncthreads();
    if (t < R) {
      double Z = 0.0;
      for (int s2 = 0; s2 < S; ++s2) Z += L.cell_z[t * S + s2];
      L.row_zk[t] = Z;
    }
  } else if (t < R) {  // many splits: one lane per row
    const size_t g0 = (size_t)global_row(t) * S;
    bool ok = true;
    float M = -INFINITY;
    for (int s2 = 0; s2 < S && ok; ++s2) {
      float m;
      double z;
      ok = read_cell(part_m, part_z, g0 + s2, epoch, &m, &z);
      M = fmaxf(M, m);
    }
    double Z = 0.0;
    for (int s2 = 0; s2 < S && ok; ++s2) {
      float m;
      double z;
      ok = read_cell(part_m, part_z, g0 + s2, epoch, &m, &z);
      if (m > -INFINITY) Z += z * exp2(((double)m - (double)M) * k64);
    }
    if (!ok) *flag = 0;
    L.row_m[t] = M;
    L.row_tau[t] = -INFINITY;
    L.row_zk[t] = Z;
  }
  __syncthreads();
  if (t < 64) {
    const int i = t;
    bool accept = false;
    if (i < K) {
      const double p = prob_at(lt, L.row_m[i], L.row_tau[i], L.row_zk[i], k64);
      const double q = prob_at(ld, L.row_m[K + 1 + i], L.row_tau[K + 1 + i], L.row_zk[K + 1 + i], k64);
      accept = (double)u_accept[(size_t)b * K + i] * q < p;
      if (write_outputs && out_p) out_p[(size_t)b * K + i] = (float)p;
      if (write_outputs && out_q) out_q[(size_t)b * K + i] = (float)q;
    }
    const uint64_t acc = __ballot(accept);
    const uint64_t live = K >= 64 ? ~0ull : ((1ull << K) - 1ull);
    const uint64_t rej = ~acc & live;
    const int n = rej ? __builtin_ctzll(rej) : K;
    if (write_outputs) {
      if (i <= K && i != n) out_tokens[(size_t)b * (K + 1) + i] = i < n ? x : -1;
      if (i == 0) out_accepted[b] = n;
    }
    if (i == n) {
      Decision d;
      d.n = n;
      d.mode = n < K ? kModeResidual : kModeBonus;
      d.m_t = L.row_m[n];
      d.tau_t = L.row_tau[n];
      d.inv_t = 1.0 / L.row_zk[n];
      const int dr = n < K ? K + 1 + n : n;  // bonus: the draft terms repeat the target's
      d.m_d = L.row_m[dr];
      d.tau_d = L.row_tau[dr];
      d.inv_d = n < K ? 1.0 / L.row_zk[dr] : 0.0;
      *sd = d;
    }
  }
  __syncthreads();
  return *flag != 0;
}

// One residual split in registers: the 16-byte groups of target row n and
// draft row n, their masses per group, and the scalar head / tail (lane 0).
template <int DT>
struct SplitRegs {
  Span st, sq;
  int head, nvec, tail0;
  bool aligned;
  u32x4 wt[kVecPerThreadB], wq[kVecPerThreadB];
  double cr[kVecPerThreadB], cp[kVecPerThreadB];
  double hr, hp, tr, tp;
  int lr, lp;  // split-relative last element with r > 0 / p' > 0 (this lane)
};

template <int DT>
__device__ __forceinline__ void load_split(SplitRegs<DT> &X, const char *rt, const char *rd, int V,
                                           int s, const Decision &d, Scale k) {
  constexpr int EPV = 16 / elem_bytes(DT);
  constexpr int VB = kVecPerThreadB;
  const int t = threadIdx.x;
  X.st = split_span_n(rt, V, s, split_elems_b(DT), DT);
  X.sq = split_span_n(rd, V, s, split_elems_b(DT), DT);
  X.aligned = X.st.head == X.sq.head;
  X.head = X.aligned ? X.st.head : 0;
  X.nvec = X.aligned ? X.st.nvec : X.st.n / EPV;
  X.tail0 = X.head + X.nvec * EPV;
  const int es = elem_bytes(DT);
  // All loads are issued before any is used: lanes past the body re-read its
  // last group (never used), so no load sits behind a select or a branch.
  if (X.nvec > 0) {
    const int last = X.nvec - 1;
    if (X.aligned) {
      const u32x4 *bt = reinterpret_cast<const u32x4 *>(X.st.base + (size_t)X.head * es);
      const u32x4 *bq = reinterpret_cast<const u32x4 *>(X.sq.base + (size_t)X.head * es);
#pragma unroll
      for (int u = 0; u < VB; ++u) {
        const int v = min(t + u * kThreads, last);
        X.wt[u] = bt[v];
        X.wq[u] = bq[v];
      }
    } else {
#pragma unroll
      for (int u = 0; u < VB; ++u) {
        const int v = min(t + u * kThreads, last);
        const size_t off = (size_t)(X.head + v * EPV) * es;
        X.wt[u] = load_group<DT>(X.st.base + off, false);
        X.wq[u] = load_group<DT>(X.sq.base + off, false);
      }
    }
  }
  X.lr = -1;
  X.lp = -1;
#pragma unroll
  for (int u = 0; u < VB; ++u) {
    X.cr[u] = 0.0;
    X.cp[u] = 0.0;
    const int v = t + u * kThreads;
    if (v < X.nvec) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        double r, p;
        resid_terms(vec_elem(X.wt[u], e, DT), vec_elem(X.wq[u], e, DT), d, k, r, p);
        X.cr[u] += r;
        X.cp[u] += p;
        const int j = X.head + v * EPV + e;
        X.lr = r > 0.0 ? j : X.lr;
        X.lp = p > 0.0 ? j : X.lp;
      }
    }
  }
  X.hr = X.hp = X.tr = X.tp = 0.0;
  if (t == 0) {
    for (int j = 0; j < X.head; ++j) {
      double r, p;
      resid_terms(load_elem(X.st.base, j, DT), load_elem(X.sq.base, j, DT), d, k, r, p);
      X.hr += r;
      X.hp += p;
      if (r > 0.0) X.lr = max(X.lr, j);
      if (p > 0.0) X.lp = max(X.lp, j);
    }
    for (int j = X.tail0; j < X.st.n; ++j) {
      double r, p;
      resid_terms(load_elem(X.st.base, j, DT), load_elem(X.sq.base, j, DT), d, k, r, p);
      X.tr += r;
      X.tp += p;
      if (r > 0.0) X.lr = max(X.lr, j);
      if (p > 0.0) X.lp = max(X.lp, j);
    }
  }
}

// Within a split held in registers: the first element whose cumulative mass
// exceeds `rem` (entries [head | groups | tail] are scanned in id order);
// split-relative, -1 if rounding left no crossing.  Whole workgroup.
template <int DT>
__device__ __forceinline__ int draw_in_split(const SplitRegs<DT> &X, double rem, bool use_p, const Decision &d,
                             Scale k, DrawLds &D) {
  constexpr int EPV = 16 / elem_bytes(DT);
  constexpr int VB = kVecPerThreadB;
  const int t = threadIdx.x;
  __shared__ int s_entry, s_token;
  __shared__ double s_before;
  const int nvec = X.nvec;
  const int E = nvec + 2;
#pragma unroll
  for (int u = 0; u < VB; ++u) {
    const int v = t + u * kThreads;
    if (v < nvec) D.val[1 + v] = use_p ? X.cp[u] : X.cr[u];
  }
  if (t == 0) {
    D.val[0] = use_p ? X.hp : X.hr;
    D.val[1 + nvec] = use_p ? X.tp : X.tr;
    s_entry = kNoEntry;
    s_token = -1;
  }
  __syncthreads();
  const int per = (E + kThreads - 1) / kThreads;
  const int e0 = min(E, t * per), e1 = min(E, e0 + per);
  double own = 0.0;
  for (int e = e0; e < e1; ++e) own += D.val[e];
  D.tsum[t] = own;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const double v = t >= off ? D.tsum[t - off] : 0.0;
    __syncthreads();
    D.tsum[t] += v;
    __syncthreads();
  }
  {
    double c = t > 0 ? D.tsum[t - 1] : 0.0;
    for (int e = e0; e < e1; ++e) {
      const double v = D.val[e];
      if (c <= rem && rem < c + v) atomicMin(&s_entry, e);  // lowest entry wins
      c += v;
    }
  }
  __syncthreads();
  const int ent = s_entry;
  if (ent != kNoEntry && t == 0) {  // the winner's base, summed in the same order
    const int owner = ent / per;
    double cc = owner > 0 ? D.tsum[owner - 1] : 0.0;
    for (int e = owner * per; e < ent; ++e) cc += D.val[e];
    s_before = cc;
  }
  __syncthreads();
  auto value = [&](float a, float q) {
    double r, p;
    resid_terms(a, q, d, k, r, p);
    return use_p ? p : r;
  };
  if (ent != kNoEntry) {
    const double before = s_before;
    if (ent == 0 || ent == nvec + 1) {  // the scalar head or tail
      if (t == 0) {
        const int j0 = ent == 0 ? 0 : X.tail0, j1 = ent == 0 ? X.head : X.st.n;
        double cc = before;
        int pick = -1, last_pos = -1;
        for (int j = j0; j < j1 && pick < 0; ++j) {
          const double v = value(load_elem(X.st.base, j, DT), load_elem(X.sq.base, j, DT));
          if (v > 0.0) last_pos = j;
          cc += v;
          if (cc > rem) pick = j;
        }
        s_token = pick >= 0 ? pick : last_pos;
      }
    } else {
      const int v = ent - 1;
      if (t == v % kThreads) {
        const int uu = v / kThreads;
        double cc = before;
        int pick = -1, last_pos = -1;
        // constant register indexes only: the scan is unrolled per group slot
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          if (u == uu) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
              const double val = value(vec_elem(X.wt[u], e, DT), vec_elem(X.wq[u], e, DT));
              const int j = X.head + v * EPV + e;
              if (pick < 0) {
                if (val > 0.0) last_pos = j;
                cc += val;
                if (cc > rem) pick = j;
              }
            }
          }
        }
        s_token = pick >= 0 ? pick : last_pos;
      }
    }
  }
  __syncthreads();
  return s_token;
}

template <int DT>
__device__ void residual_tile(const char *target, const char *draft, const int32_t *tokens,
                              const float *u_accept, const float *u_sample, int B, int K, int V,
                              int S, int SB, double k64, Scale k, u64 epoch,
                              const u64 *part_m, const u64 *part_z, const u64 *part_x,
                              const RowStat *rowstat, ResidPart *rpart, int32_t *out_accepted,
                              int32_t *out_tokens, float *out_p, float *out_q, float *out_mass,
                              int b, int s) {
  const int t = threadIdx.x;
  __shared__ TileLds lds;
  __shared__ Decision sdec;
  __shared__ int s_ok, s_split, s_use_p, s_fb_token;
  __shared__ double s_rem, s_total;
  __shared__ double red_r[kThreads / 64], red_p[kThreads / 64];
  __shared__ int red_lr[kThreads / 64], red_lp[kThreads / 64];

  // 1. decide, once every streaming tile of request b has published
  if (!decide(tokens, u_accept, B, K, S, k64, part_m, part_z, part_x, epoch,
                  rowstat, b, s == 0, out_accepted, out_tokens, out_p, out_q, lds.dec, &sdec,
                  &s_ok)) {
    if (t == 0) out_accepted[b] = -2;  // time-out: flag the request as failed
    return;
  }
  const Decision d = sdec;
  const char *rt = row_ptr(target, (size_t)b * (K + 1) + d.n, V, DT);
  const char *rd = d.mode == kModeResidual ? row_ptr(draft, (size_t)b * K + d.n, V, DT) : rt;

  // 2. the residual mass of split s, published as one record
  {
    SplitRegs<DT> X;
    load_split<DT>(X, rt, rd, V, s, d, k);
    double own_r = X.hr + X.tr, own_p = X.hp + X.tp;
#pragma unroll
    for (int u = 0; u < kVecPerThreadB; ++u) {
      own_r += X.cr[u];
      own_p += X.cp[u];
    }
    own_r = wave_sum(own_r);
    own_p = wave_sum(own_p);
    int wl_r = X.lr, wl_p = X.lp;
    for (int o = 32; o > 0; o >>= 1) {
      wl_r = max(wl_r, __shfl_xor(wl_r, o, 64));
      wl_p = max(wl_p, __shfl_xor(wl_p, o, 64));
    }
    if (lane_id() == 0) {
      red_r[t >> 6] = own_r;
      red_p[t >> 6] = own_p;
      red_lr[t >> 6] = wl_r;
      red_lp[t >> 6] = wl_p;
    }
    __syncthreads();
    if (t == 0) {
      double R2 = 0.0, P2 = 0.0;
      int LR = -1, LP = -1;
      for (int w = 0; w < kThreads / 64; ++w) {
        R2 += red_r[w];
        P2 += red_p[w];
        LR = max(LR, red_lr[w]);
        LP = max(LP, red_lp[w]);
      }
      ResidPart *out = rpart + (size_t)b * SB + s;
      store_agent(&out->r, pack_f64(R2, epoch));
      store_agent(&out->p, pack_f64(P2, epoch));
      store_agent(&out->idx, pack_idx2(LR, LP, epoch));
    }
  }
  // only the request's last residual tile (dispatched after its siblings)
  // gathers the split masses and draws
  if (s != SB - 1) return;

  // 3. the draw: which split holds u * S?
  DrawLds &D = lds.draw;
  {
    bool ok = true;
    const ResidPart *rp = rpart + (size_t)b * SB;
    for (int i = t; i < SB; i += kThreads) {
      bool got = false;
      for (int it = 0; it < kSpinLimit && !got; ++it) {
        const u64 rw = load_agent(&rp[i].r), pw = load_agent(&rp[i].p), iw = load_agent(&rp[i].idx);
        double rv, pv;
        int a, c;
        got = unpack_f64(rw, epoch, &rv) & unpack_f64(pw, epoch, &pv) & unpack_idx2(iw, epoch, &a, &c);
        if (got) {
          D.pr[i] = rv;
          D.pp[i] = pv;
          D.plr[i] = a >= 0 ? i * split_elems_b(DT) + a : -1;
          D.plp[i] = c >= 0 ? i * split_elems_b(DT) + c : -1;
        } else {
          spin_pause();
        }
      }
      ok = ok && got;
    }
    if (t == 0) s_ok = 1;
    __syncthreads();
    if (!ok) s_ok = 0;
    __syncthreads();
    if (!s_ok) {
      if (t == 0) out_accepted[b] = -2;
      return;
    }
  }
  if (t == 0) {
    double Sr = 0.0;
    for (int i = 0; i < SB; ++i) Sr += D.pr[i];
    int use_p = 0;
    double tot = Sr;
    if (!(Sr > 0.0)) {  // unreachable in exact arithmetic after a rejection
      use_p = 1;
      tot = 0.0;
      for (int i = 0; i < SB; ++i) tot += D.pp[i];
    }
    const double goal = (double)u_sample[b] * tot;
    double c = 0.0;
    int split = -1;
    for (int i = 0; i < SB; ++i) {
      const double v = use_p ? D.pp[i] : D.pr[i];
      if (c + v > goal) {
        split = i;
        break;
      }
      c += v;
    }
    int fb = -1;  // rounding left no crossing: the last token with mass
    if (split < 0)
      for (int i = SB - 1; i >= 0 && fb < 0; --i) fb = use_p ? D.plp[i] : D.plr[i];
    s_split = split;
    s_use_p = use_p;
    s_rem = goal - c;
    s_total = tot;
    s_fb_token = split >= 0 ? (use_p ? D.plp[split] : D.plr[split]) : fb;
  }
  __syncthreads();
  const int split = s_split;
  int tok = s_fb_token;
  if (split >= 0) {
    // the crossing split is read again (it is this tile's own split only one
    // time in SB; keeping that one in registers would cost every tile of the
    // kernel occupancy)
    SplitRegs<DT> Y;
    load_split<DT>(Y, rt, rd, V, split, d, k);
    const int local = draw_in_split<DT>(Y, s_rem, s_use_p != 0, d, k, D);
    if (local >= 0) tok = Y.st.e0 + local;
  }
  if (t == 0) {
    out_tokens[(size_t)b * (K + 1) + d.n] = tok;
    if (out_mass) out_mass[b] = (float)s_total;
  }
}

}  // namespace

template <int DT>
__global__ __launch_bounds__(kThreads) void k_sample_fused(
    const char *__restrict__ target, const char *__restrict__ draft,
    const int32_t *__restrict__ tokens, const float *__restrict__ u_accept,
    const float *__restrict__ u_sample, int B, int K, int V, int S, int SB, double k64, Scale k,
    u64 epoch, int phase, int lag, u64 *__restrict__ part_m, u64 *__restrict__ part_z,
    u64 *__restrict__ part_x, const RowStat *__restrict__ rowstat, ResidPart *__restrict__ rpart,
    int32_t *__restrict__ out_accepted, int32_t *__restrict__ out_tokens,
    float *__restrict__ out_p, float *__restrict__ out_q, float *__restrict__ out_mass) {
  const int blk = (int)blockIdx.x;
  const int R = 2 * K + 1;
  const int nA_req = R * S;
  bool streaming;
  int b, idx;
  if (phase == 1) {  // streaming tiles only
    streaming = true;
    b = blk / nA_req;
    idx = blk - b * nA_req;
  } else if (phase == 2) {  // residual tiles only
    streaming = false;
    b = blk / SB;
    idx = blk - b * SB;
  } else {  // group g holds [streaming(g) | residual(g - lag)]
    auto prefix = [&](int g) { return nA_req * min(g, B) + SB * min(max(g - lag, 0), B); };
    int lo = 0, hi = B + lag;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (prefix(mid) <= blk) lo = mid; else hi = mid;
    }
    const int off = blk - prefix(lo);
    const int a_here = lo < B ? nA_req : 0;
    streaming = off < a_here;
    b = streaming ? lo : lo - lag;
    idx = streaming ? off : off - a_here;
  }
  if (streaming) {
    const int r = idx / S;
    const int s = idx - r * S;
    const int rows_t = B * (K + 1);
    const int grow = r <= K ? b * (K + 1) + r : rows_t + b * K + (r - K - 1);
    const char *rp = r <= K ? row_ptr(target, (size_t)grow, V, DT)
                            : row_ptr(draft, (size_t)(grow - rows_t), V, DT);
    // the draft token's logit, if this split holds it (or, for a token out
    // of range, split 0 publishes -inf: probability 0, the draft is rejected)
    // (uniform across the workgroup: scalar registers, no vector registers
    // held across the stream)
    const int pos = r <= K ? r : r - K - 1;  // position; target row K has no draft token
    bool mine = false, valid = false;
    unsigned mis = 0;
    uint32_t w = 0;
    if (r != K) {
      const int x = tokens[(size_t)b * K + pos];
      const int e0 = s * split_elems(DT), e1 = min(V, e0 + split_elems(DT));
      valid = x >= 0 && x < V;
      mine = (valid && x >= e0 && x < e1) || (!valid && s == 0);
      if (mine && valid) {
        // the aligned dword holding the element (same page, so always
        // readable); its bits are picked apart only after the stream
        // the logits are read-only for the whole call: a scalar load through
        // the constant address space, which leaves the vector queue to the
        // stream
        typedef const __attribute__((address_space(4))) uint32_t *const_u32p;
        const uintptr_t ea = reinterpret_cast<uintptr_t>(rp) + (uintptr_t)x * elem_bytes(DT);
        mis = (unsigned)(ea & 3u);
        w = *(const_u32p)(ea - mis);
      }
    }
    float M;
    double Z;
    softmax_tile<DT>(rp, V, s, k, &M, &Z);
    if (threadIdx.x == 0) {
      store_agent(&part_m[(size_t)grow * S + s], pack_f32(M, epoch));
      store_agent(&part_z[(size_t)grow * S + s], pack_f64(Z, epoch));
      if (mine) {
        const uint32_t lx_bits = !valid ? 0xFF800000u  // -inf
                                 : DT == kBF16 ? (mis ? (w & 0xFFFF0000u) : (w << 16)) : w;
        store_agent(part_x + ((size_t)b * K + pos) * 2 + (r <= K ? 0 : 1),
                    pack_u32(lx_bits, epoch));
      }
    }
    return;
  }
  residual_tile<DT>(target, draft, tokens, u_accept, u_sample, B, K, V, S, SB, k64, k, epoch,
                    part_m, part_z, part_x, rowstat, rpart, out_accepted, out_tokens, out_p,
                    out_q, out_mass, b, idx);
}

hipError_t launch_sample(const void *target, const void *draft, int dtype, const int32_t *tokens,
                         const float *u_accept, const float *u_sample, int B, int K, int V,
                         int S, int SB, double k64, Scale k, u64 epoch, int phase, int lag,
                         u64 *part_m, u64 *part_z, u64 *part_x, const RowStat *rowstat,
                         ResidPart *rpart, int32_t *out_accepted, int32_t *out_tokens,
                         float *out_p, float *out_q, float *out_mass, hipStream_t stream) {
  const int nA = B * (2 * K + 1) * S;
  const int nB = B * SB;
  // phase: 0 = whole call, 1 = streaming tiles only, 2 = residual tiles only
  const int blocks = phase == 0 ? nA + nB : phase == 1 ? nA : nB;
  lag = std::max(1, std::min(lag, B));
  if (dtype == kBF16)
    hipLaunchKernelGGL(k_sample_fused<kBF16>, dim3(blocks), dim3(kThreads), 0, stream,
                       (const char *)target, (const char *)draft, tokens, u_accept, u_sample, B,
                       K, V, S, SB, k64, k, epoch, phase, lag, part_m, part_z, part_x, rowstat,
                       rpart, out_accepted, out_tokens, out_p, out_q, out_mass);
  else
    hipLaunchKernelGGL(k_sample_fused<kF32>, dim3(blocks), dim3(kThreads), 0, stream,
                       (const char *)target, (const char *)draft, tokens, u_accept, u_sample, B,
                       K, V, S, SB, k64, k, epoch, phase, lag, part_m, part_z, part_x, rowstat,
                       rpart, out_accepted, out_tokens, out_p, out_q, out_mass);
  return hipGetLastError();
}

// Workgroups of the fused kernel that fit on the device at once.
int resident_workgroups(int dtype) {
  static int cache[2] = {0, 0};
  const int d = dtype == kBF16 ? 1 : 0;
  if (!cache[d]) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 2048;
    const void *fn = d ? (const void *)k_sample_fused<kBF16> : (const void *)k_sample_fused<kF32>;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess)
      per_cu = 4;
    cache[d] = std::max(1, cus * per_cu);
  }
  return cache[d];
}

}  // namespace sv
