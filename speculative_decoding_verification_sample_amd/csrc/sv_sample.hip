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
// Streaming tile: the split's (max, tempered mass) partial, three words (the
// maximum, and the mass as fp32 hi + lo, each word tagged on its own).
// Residual tile (b, s), once request b's rows are all streamed:
//  1. decide: combine the (2K+1) x S partials, evaluate p'(x_i), q'(x_i) in
//     fp64 and the test u_i * q'(x_i) < p'(x_i); a ballot gives the first
//     rejection n (ariser.io review, section "같은 분포를 지키는 작은 장치":
//     accept with probability min(1, p/q); lotook.com explainer, four steps:
//     scan left to right, stop at the first mismatch).  Split 0 writes the
//     accepted drafts.
//  2. sum the residual mass max(0, p'_n - q'_n) over the split (p'_K when all
//     K drafts survived: the bonus token), fp32 terms into fp64, and publish
//     the split's total.
//  3. every residual tile of the request waits for all the split totals and
//     finds the split where the cumulative mass passes u * S (inverse CDF
//     over ascending ids); that split's tile scans its per-lane masses and
//     one wave walks to the token, re-reading what the tile itself just read
//     (its own L2).  The other tiles exit.
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

// LDS shared by the decide and draw phases of a residual tile.
struct DecideLds {
  float cell_m[kMaxCells];
  double cell_z[kMaxCells];
  float row_m[128], row_tau[128];
  double row_zk[128];
};
struct DrawLds {
  double tot[kMaxSplitsB];  // split masses of the request
  double wsum[kThreads / 64], wprev[kThreads / 64], lanes_end;
  double eh, et;  // the split's scalar head and tail masses
  int wfirst[kThreads / 64], wlast[kThreads / 64];
};
union TileLds {
  DecideLds dec;
  DrawLds draw;
};
// Everything a residual tile keeps in LDS (one allocation for the kernel).
struct ResidLds {
  TileLds lds;
  Decision dec;
  int ok, split, use_p;
  double rem, total;
  double red[kThreads / 64];
};

// p'(x) of one row at logit l (fp64): zero outside the nucleus.
__device__ __forceinline__ double prob_at(float l, float m, float tau, double zk, double k64) {
  if (!(l >= tau)) return 0.0;
  return exp2(((double)l - (double)m) * k64) / zk;
}

// Mass of one token of the drawn row pair: the residual r = max(0, p' - q')
// (the bonus draw has inv_d = 0, so r = p'), or p' itself (P: the fallback
// when the residual mass is not positive).  Every pass over the pair computes
// it with this one function, so the values agree bit for bit.  fp32 terms
// 2^((l - m) k) times the inverse kept mass as a float pair (one fused
// multiply-add: the product carries one rounding, and no common factor
// separates p' from q'); the difference in fp32, the sums over a split in
// fp64.
template <bool TOPP, bool P>
__device__ __forceinline__ double token_mass(float lt, float ld, const Decision &d, Scale k) {
  const float et = tempered(lt, d.m_t, k);
  float pt = fmaf(et, d.inv_t, et * d.inv_t_lo);
  if (TOPP) pt = lt >= d.tau_t ? pt : 0.f;
  if (P) return (double)pt;
  const float ed = tempered(ld, d.m_d, k);
  float qd = fmaf(ed, d.inv_d, ed * d.inv_d_lo);
  if (TOPP) qd = ld >= d.tau_d ? qd : 0.f;
  return (double)fmaxf(pt - qd, 0.f);
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

// Lanes per row group in the decide: S rounded up to a power of two.
__device__ __forceinline__ int group_lanes(int S) {
  return S <= 1 ? 1 : S <= 2 ? 2 : S <= 4 ? 4 : S <= 8 ? 8 : 16;
}

// Maximum / fp64 sum over aligned groups of G lanes (G in 1, 2, 4, 8, 16),
// valid in every lane of the group.  Every lane must be active.
__device__ __forceinline__ float group_max(float v, int G) {
  const uint32_t id = __float_as_uint(-INFINITY);
  if (G >= 2) v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor1>(id, __float_as_uint(v))));
  if (G >= 4) v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor2>(id, __float_as_uint(v))));
  if (G >= 8) v = fmaxf(v, __uint_as_float(dpp_u32<kDppHalfMirror>(id, __float_as_uint(v))));
  if (G >= 16) v = fmaxf(v, __uint_as_float(dpp_u32<kDppMirror>(id, __float_as_uint(v))));
  return v;
}
__device__ __forceinline__ double group_sum(double v, int G) {
  auto bits = [](double x) { return (uint64_t)__double_as_longlong(x); };
  auto val = [](uint64_t x) { return __longlong_as_double((long long)x); };
  if (G >= 2) v += val(dpp_u64<kDppXor1>(0, bits(v)));
  if (G >= 4) v += val(dpp_u64<kDppXor2>(0, bits(v)));
  if (G >= 8) v += val(dpp_u64<kDppHalfMirror>(0, bits(v)));
  if (G >= 16) v += val(dpp_u64<kDppMirror>(0, bits(v)));
  return v;
}

// Poll one (row, split) cell until it carries this call's epoch.
__device__ __forceinline__ bool read_cell(const u64 *part_m, const u64 *part_z, size_t g,
                                          u64 epoch, float *m, double *z) {
  for (int it = 0; it < kSpinLimit; ++it) {
    const u64 mw = load_agent(&part_m[g]);
    const u64 hw = load_agent(&part_z[2 * g]);
    const u64 lw = load_agent(&part_z[2 * g + 1]);
    uint32_t mb, hb, lb;
    if ((int)unpack_u32(mw, epoch, &mb) & (int)unpack_u32(hw, epoch, &hb) &
        (int)unpack_u32(lw, epoch, &lb)) {
      *m = __uint_as_float(mb);
      *z = (double)__uint_as_float(hb) + (double)__uint_as_float(lb);
      return true;
    }
    spin_pause();
  }
  return false;
}

// The accept / reject outcome of request b into *sd; whole workgroup.
// Returns false if a partial never arrived (bounded wait timed out).
__device__ __forceinline__ bool decide(const int32_t *tokens, const float *u_accept, int B, int K, int S,
                       double k64, Scale k, const u64 *part_m, const u64 *part_z,
                       const u64 *part_x, u64 epoch,
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
  float lt = -INFINITY, ld = -INFINITY, ua = 0.f;
  bool got_x = true;
  if (t < K) {
    x = tokens[(size_t)b * K + t];
    ua = u_accept[(size_t)b * K + t];  // issued early: off the critical path
    const u64 *px = part_x + ((size_t)b * K + t) * 2;
    got_x = false;
    for (int it = 0; it < kSpinLimit && !got_x; ++it) {
      uint32_t bt, bd;
      got_x = ((int)unpack_u32(load_agent(&px[0]), epoch, &bt) &
               (int)unpack_u32(load_agent(&px[1]), epoch, &bd)) != 0;
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
  } else if (S <= 16 && R * group_lanes(S) <= kThreads) {
    // one lane per cell, a row's cells in a group of G lanes (S rounded up
    // to a power of two): the row's maximum and mass by lane moves inside
    // the group, no pass over LDS
    const int G = group_lanes(S);
    const int r = t / G, c = t - r * G;
    float m = -INFINITY;
    double z = 0.0;
    if (r < R && c < S &&
        !read_cell(part_m, part_z, (size_t)global_row(r) * S + c, epoch, &m, &z))
      *flag = 0;
    const float M = group_max(m, G);
    const double Z = group_sum(m > -INFINITY ? z * exp2(((double)m - (double)M) * k64) : 0.0, G);
    if (r < R && c == 0) {
      L.row_m[r] = M;
      L.row_tau[r] = -INFINITY;
      L.row_zk[r] = Z;
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
      accept = (double)ua * q < p;
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
      split_f64(1.0 / L.row_zk[n], &d.inv_t, &d.inv_t_lo);
      if (n < K) {
        d.m_d = L.row_m[K + 1 + n];
        d.tau_d = L.row_tau[K + 1 + n];
        split_f64(1.0 / L.row_zk[K + 1 + n], &d.inv_d, &d.inv_d_lo);
      } else {  // bonus: no draft row; its weight 0 makes the residual p'
        d.m_d = d.m_t;
        d.tau_d = d.tau_t;
        d.inv_d = 0.f;
        d.inv_d_lo = 0.f;
      }
      *sd = d;
    }
  }
  __syncthreads();
  return *flag != 0;
}

// ---------------------------------------------------------------------------
// residual (or bonus) draw
// ---------------------------------------------------------------------------

// One residual split of the drawn row pair.  Lane t owns body groups
// [t VB, t VB + VB) (consecutive, so a lane's entry is a run of token ids).
struct SplitGeo {
  const char *bt, *bq;  // element 0 of the split in the target / draft row
  int e0, n;            // first element (row-relative) and elements in the split
  int head, nvec, tail0;  // scalar head, 16-byte groups, first tail element
  bool aligned;           // both rows share the 16-byte phase: vector loads
};

template <int DT>
__device__ __forceinline__ SplitGeo split_geo(const char *rt, const char *rd, int V, int s) {
  constexpr int EPV = 16 / elem_bytes(DT);
  const Span a = split_span_n(rt, V, s, split_elems_b(DT), DT);
  const Span q = split_span_n(rd, V, s, split_elems_b(DT), DT);
  SplitGeo g;
  g.bt = a.base;
  g.bq = q.base;
  g.e0 = a.e0;
  g.n = a.n;
  g.aligned = a.head == q.head;
  g.head = g.aligned ? a.head : 0;  // misaligned pair: groups assembled from scalars
  g.nvec = g.aligned ? a.nvec : a.n / EPV;
  g.tail0 = g.head + g.nvec * EPV;
  return g;
}

// Split-relative element range [j0, j1) of entry `ent`.
template <int DT>
__device__ __forceinline__ void entry_range(const SplitGeo &g, int ent, int &j0, int &j1) {
  constexpr int EPV = 16 / elem_bytes(DT);
  constexpr int VB = kVecPerThreadB;
  if (ent == 0) {
    j0 = 0;
    j1 = g.head;
  } else if (ent == kThreads + 1) {
    j0 = g.tail0;
    j1 = g.n;
  } else {
    j0 = g.head + min((ent - 1) * VB, g.nvec) * EPV;
    j1 = g.head + min(ent * VB, g.nvec) * EPV;
  }
}

// This lane's body groups of the drawn row pair: kVecPerThreadB consecutive
// 16-byte groups of each row.  All loads are issued before any is used; lanes past the body re-read
// its last group (never used).  P: the target row only.
struct LaneGroups {
  u32x4 wt[kVecPerThreadB], wq[kVecPerThreadB];
};

template <int DT, bool P>
__device__ __forceinline__ void load_lane(const SplitGeo &g, LaneGroups &L) {
  constexpr int EPV = 16 / elem_bytes(DT);
  constexpr int VB = kVecPerThreadB;
  if (g.nvec <= 0) return;
  const int v0 = threadIdx.x * VB;
  const int last = g.nvec - 1;
  const int es = elem_bytes(DT);
  if (g.aligned) {
    const u32x4 *pt = reinterpret_cast<const u32x4 *>(g.bt + (size_t)g.head * es);
    const u32x4 *pq = reinterpret_cast<const u32x4 *>(g.bq + (size_t)g.head * es);
#pragma unroll
    for (int u = 0; u < VB; ++u) {
      const int v = min(v0 + u, last);
      L.wt[u] = pt[v];
      if (!P) L.wq[u] = pq[v];
    }
  } else {
#pragma unroll
    for (int u = 0; u < VB; ++u) {
      const size_t off = (size_t)min(v0 + u, last) * EPV * es;
      L.wt[u] = load_group<DT>(g.bt + off, false);
      if (!P) L.wq[u] = load_group<DT>(g.bq + off, false);
    }
  }
}

// Mass of this lane's body entry, in element order.
template <int DT, bool TOPP, bool P>
__device__ __forceinline__ double lane_mass(const SplitGeo &g, const LaneGroups &L,
                                            const Decision &d, Scale k) {
  constexpr int EPV = 16 / elem_bytes(DT);
  constexpr int VB = kVecPerThreadB;
  const int v0 = threadIdx.x * VB;
  double acc = 0.0;
#pragma unroll
  for (int u = 0; u < VB; ++u) {
    if (v0 + u < g.nvec) {
#pragma unroll
      for (int e = 0; e < EPV; ++e)
        acc += token_mass<TOPP, P>(vec_elem(L.wt[u], e, DT), P ? 0.f : vec_elem(L.wq[u], e, DT), d, k);
    }
  }
  return acc;
}

// Mass of split-relative elements [j0, j1), one lane, scalar loads.
template <int DT, bool TOPP, bool P>
__device__ __forceinline__ double range_mass(const SplitGeo &g, int j0, int j1, const Decision &d,
                                             Scale k) {
  double acc = 0.0;
  for (int j = j0; j < j1; ++j)
    acc += token_mass<TOPP, P>(load_elem(g.bt, j, DT), P ? 0.f : load_elem(g.bq, j, DT), d, k);
  return acc;
}

// Sum over the workgroup (valid in every thread); `red` holds kThreads / 64.
__device__ __forceinline__ double block_sum(double v, double *red) {
  v = wave_sum(v);
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

// Cumulative masses of a split's entries from the start of the split: this
// lane's entry ends at `incl` and starts at `prev`.
struct SplitScan {
  double prev, incl;
};

// The scan part of the draw, which does not need the target u * S yet.
// Whole workgroup; sets D.lanes_end.
__device__ __forceinline__ SplitScan scan_split(double e_head, double e_lane, DrawLds &D) {
  const int l = lane_id(), w = threadIdx.x >> 6;
  const double incl_w = wave_incl_scan(e_lane);
  const double up = __shfl_up(incl_w, 1, 64);
  if (l == 63) D.wsum[w] = incl_w;
  __syncthreads();
  double off = e_head;
  for (int i = 0; i < w; ++i) off += D.wsum[i];
  SplitScan r;
  r.incl = off + incl_w;
  r.prev = l > 0 ? off + up : off;
  if (threadIdx.x == kThreads - 1) D.lanes_end = r.incl;
  __syncthreads();
  return r;
}

// The draw inside one split: entries (head, lanes, tail) with masses e_head,
// e_lane (this thread's lane entry, scanned into `sc`) and e_tail; the
// token is the first one whose cumulative mass from the start of the split
// exceeds `rem`.  Returns the split-relative token in every thread; if
// rounding leaves no crossing, the last token with positive mass.  Whole
// workgroup.
template <int DT, bool TOPP, bool P>
__device__ __forceinline__ int draw_split(const SplitGeo &g, double e_head, double e_lane,
                                          double e_tail, const SplitScan &sc, double rem,
                                          const Decision &d, Scale k, DrawLds &D) {
  __shared__ int s_ent;
  __shared__ double s_base;
  const int t = threadIdx.x, l = lane_id(), w = t >> 6;
  // 1. the crossing entry: cumulative masses head, lanes 0..255, tail
  const double prev = sc.prev, incl = sc.incl;
  const uint64_t cross = __ballot(prev <= rem && rem < incl);
  const uint64_t pos = __ballot(e_lane > 0.0);
  if (l == 0) {
    D.wfirst[w] = cross ? w * 64 + __builtin_ctzll(cross) : -1;
    D.wlast[w] = pos ? w * 64 + 63 - __builtin_clzll(pos) : -1;
  }
  if (cross && l == __builtin_ctzll(cross)) D.wprev[w] = prev;
  __syncthreads();
  if (t == 0) {
    int ent = -1;
    double base = 0.0;
    if (rem < e_head) {
      ent = 0;
    } else {
      for (int i = 0; i < kThreads / 64 && ent < 0; ++i)
        if (D.wfirst[i] >= 0) {
          ent = 1 + D.wfirst[i];
          base = D.wprev[i];
        }
      if (ent < 0 && rem < D.lanes_end + e_tail) {
        ent = kThreads + 1;
        base = D.lanes_end;
      }
    }
    if (ent < 0) {  // rounding: no crossing; the last entry with mass, walked to its end
      if (e_tail > 0.0) ent = kThreads + 1;
      for (int i = kThreads / 64 - 1; i >= 0 && ent < 0; --i)
        if (D.wlast[i] >= 0) ent = 1 + D.wlast[i];
      if (ent < 0) ent = 0;
      base = -INFINITY;  // never crosses: the walk keeps the last token with mass
    }
    s_ent = ent;
    s_base = base;
  }
  __syncthreads();
  const int ent = s_ent;
  // 2. the walk: one wave, one token per lane, an inclusive scan of the masses
  __shared__ int s_tok;
  if (w == 0) {
    int j0, j1;
    entry_range<DT>(g, ent, j0, j1);
    const int j = j0 + l;
    const bool in = j < j1;
    const double v =
        in ? token_mass<TOPP, P>(load_elem(g.bt, j, DT), P ? 0.f : load_elem(g.bq, j, DT), d, k)
           : 0.0;
    const double c = s_base + wave_incl_scan(v);
    const uint64_t hit = __ballot(in && c > rem);
    const uint64_t has = __ballot(in && v > 0.0);
    if (l == 0)
      s_tok = hit ? j0 + __builtin_ctzll(hit) : has ? j0 + 63 - __builtin_clzll(has) : -1;
  }
  __syncthreads();
  return s_tok;
}

// Inverse CDF over the split masses tot[0..SB): the split where the
// cumulative mass first exceeds u * (sum of all), and what is left of u * sum
// at its start.  If rounding leaves no crossing, the last split with mass
// and rem = +inf (its last token with mass is drawn); -1 if none has mass.
__device__ __forceinline__ int pick_split(const double *tot, int SB, float u, double *rem,
                                          double *total) {
  double sum = 0.0;
  for (int i = 0; i < SB; ++i) sum += tot[i];
  const double goal = (double)u * sum;
  double c = 0.0;
  int split = -1, last = -1;
  for (int i = 0; i < SB && split < 0; ++i) {
    if (tot[i] > 0.0) last = i;
    if (c + tot[i] > goal) split = i;
    else c += tot[i];
  }
  if (split < 0) {
    split = last;
    c = -INFINITY;
  }
  *rem = goal - c;
  *total = sum;
  return split;
}

// pick_split over SB <= 64 masses held one per lane of a wave (lane i holds
// split i, lanes >= SB hold 0), by an inclusive scan; the same outcome rule.
// The whole wave calls it; the results are valid in every lane.
__device__ __forceinline__ int pick_split_wave(double v, int SB, float u, double *rem,
                                               double *total) {
  const int l = lane_id();
  const double incl = wave_incl_scan(v);
  auto lane_val = [&](double x, int lane) {
    const long long b = __double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)b >> 32), lane);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  };
  const double sum = lane_val(incl, SB - 1);
  const double goal = (double)u * sum;
  const uint64_t hit = __ballot(l < SB && incl > goal);
  int split;
  double c;
  if (hit) {
    split = __builtin_ctzll(hit);
    c = split > 0 ? lane_val(incl, split - 1) : 0.0;
  } else {  // rounding: the last split with mass, to its end
    const uint64_t pos = __ballot(l < SB && v > 0.0);
    split = pos ? 63 - __builtin_clzll(pos) : -1;
    c = -INFINITY;
  }
  *rem = goal - c;
  *total = sum;
  return split;
}

// Residual tile (b, s).  Every tile of the request decides, sums its split's
// residual masses, publishes the split's total, and waits for all its
// siblings' totals: the one tile whose split holds u * S then draws, from
// the per-lane masses it still holds and rows it has just read.  A tile
// only waits for siblings dispatched before it or after it; those after it
// are the rest of one request, so at most SB - 1 tiles ever wait for work
// not yet dispatched, far fewer than the device holds.
template <int DT, bool TOPP>
__device__ __forceinline__ void residual_tile(const char *target, const char *draft, const int32_t *tokens,
                              const float *u_accept, const float *u_sample, int B, int K, int V,
                              int S, int SB, double k64, Scale k, u64 epoch,
                              const u64 *part_m, const u64 *part_z, const u64 *part_x,
                              const RowStat *rowstat, u64 *rtot,
                              int32_t *out_accepted, int32_t *out_tokens, float *out_p,
                              float *out_q, float *out_mass, int b, int s, ResidLds &R) {
  const int t = threadIdx.x;
  const float us = u_sample[b];  // any tile may hold the crossing; issued early
  TileLds &lds = R.lds;
  Decision &sdec = R.dec;
  int &s_ok = R.ok, &s_split = R.split, &s_use_p = R.use_p;
  double &s_rem = R.rem, &s_total = R.total;
  double *red = R.red;

  // 1. decide, once every streaming tile of request b has published
  if (!decide(tokens, u_accept, B, K, S, k64, k, part_m, part_z, part_x, epoch, rowstat, b,
              s == 0, out_accepted, out_tokens, out_p, out_q, lds.dec, &sdec, &s_ok)) {
    if (t == 0) out_accepted[b] = -2;  // time-out: flag the request as failed
    return;
  }
  const Decision d = sdec;
  const char *rt = row_ptr(target, (size_t)b * (K + 1) + d.n, V, DT);
  const char *rd = d.mode == kModeResidual ? row_ptr(draft, (size_t)b * K + d.n, V, DT) : rt;

  // 2. the residual masses of split s: the lane entries, head and tail, total
  DrawLds &D = lds.draw;
  const SplitGeo g = split_geo<DT>(rt, rd, V, s);
  LaneGroups mine;
  load_lane<DT, false>(g, mine);
  if (t == 0) {
    D.eh = range_mass<DT, TOPP, false>(g, 0, g.head, d, k);
    D.et = range_mass<DT, TOPP, false>(g, g.tail0, g.n, d, k);
  }
  const double lm = lane_mass<DT, TOPP, false>(g, mine, d, k);
  const double tot = block_sum(lm + (t == 0 ? D.eh + D.et : 0.0), red);  // syncs: D.eh / D.et visible
  // the split's mass as hi + lo fp32 halves, each word tagged with the
  // epoch's low 32 bits: a stale pair validates with probability 2^-64
  if (t == 0) {
    const float hi = (float)tot, lo = (float)(tot - (double)hi);
    store_agent(&rtot[((size_t)b * SB + s) * 2], pack_u32(__float_as_uint(hi), epoch));
    store_agent(&rtot[((size_t)b * SB + s) * 2 + 1], pack_u32(__float_as_uint(lo), epoch));
  }
  const double eh = D.eh, et = D.et;
  // the split's own scan, while the sibling totals are on their way
  const SplitScan sc = scan_split(eh, lm, D);

  // 3. every split's total; which split holds u * S?
  {
    bool ok = true;
    for (int i = t; i < SB; i += kThreads) {
      bool got = false;
      double v = 0.0;
      for (int it = 0; it < kSpinLimit && !got; ++it) {
        uint32_t hi, lo;
        got = ((int)unpack_u32(load_agent(&rtot[((size_t)b * SB + i) * 2]), epoch, &hi) &
               (int)unpack_u32(load_agent(&rtot[((size_t)b * SB + i) * 2 + 1]), epoch, &lo)) != 0;
        v = (double)__uint_as_float(hi) + (double)__uint_as_float(lo);
        if (!got) spin_pause();
      }
      D.tot[i] = v;
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
  if (SB <= 64) {  // one wave: a scan of the split masses
    if (t < 64) {
      double rem, total;
      const int split = pick_split_wave(t < SB ? D.tot[t] : 0.0, SB, us, &rem, &total);
      if (t == 0) {
        s_use_p = !(total > kResidualResolution);
        s_split = split;
        s_rem = rem;
        s_total = total;
      }
    }
  } else if (t == 0) {
    double rem, total;
    const int split = pick_split(D.tot, SB, us, &rem, &total);
    s_use_p = !(total > kResidualResolution);
    s_split = split;
    s_rem = rem;
    s_total = total;
  }
  // S = 0 cannot happen in exact arithmetic after a rejection (the residual
  // holds at least q'(x) - p'(x) > 0); it can when p' and q' agree and the
  // draft token has no mass under either.  An S at or below the resolution
  // level (rounding alone) sends the last tile to draw from p' instead
  // (recomputed split by split: rare and slow).
  __syncthreads();
  if (!s_use_p) {
    const int claim = s_split >= 0 ? s_split : SB - 1;
    if (s != claim) return;
    int tok = -1;
    if (s_split >= 0) {
      const int local = draw_split<DT, TOPP, false>(g, eh, lm, et, sc, s_rem, d, k, D);
      if (local >= 0) tok = g.e0 + local;
    }
    if (t == 0) {
      out_tokens[(size_t)b * (K + 1) + d.n] = tok;
      if (out_mass) out_mass[b] = (float)s_total;
    }
    return;
  }

  // the p' fallback, by the request's last tile
  if (s != SB - 1) return;
  for (int i = 0; i < SB; ++i) {
    const SplitGeo gi = split_geo<DT>(rt, rd, V, i);
    LaneGroups li;
    load_lane<DT, true>(gi, li);
    double v = lane_mass<DT, TOPP, true>(gi, li, d, k);
    if (t == 0)
      v += range_mass<DT, TOPP, true>(gi, 0, gi.head, d, k) +
           range_mass<DT, TOPP, true>(gi, gi.tail0, gi.n, d, k);
    v = block_sum(v, red);
    if (t == 0) D.tot[i] = v;
  }
  __syncthreads();
  if (t == 0) {
    double rem, total;
    s_split = pick_split(D.tot, SB, us, &rem, &total);
    s_rem = rem;
    s_total = total;
  }
  __syncthreads();
  int tok = -1;
  if (s_split >= 0) {
    const SplitGeo gs = split_geo<DT>(rt, rd, V, s_split);
    LaneGroups ls;
    load_lane<DT, true>(gs, ls);
    const double el = lane_mass<DT, TOPP, true>(gs, ls, d, k);
    if (t == 0) {
      D.eh = range_mass<DT, TOPP, true>(gs, 0, gs.head, d, k);
      D.et = range_mass<DT, TOPP, true>(gs, gs.tail0, gs.n, d, k);
    }
    __syncthreads();
    const double eh2 = D.eh, et2 = D.et;
    const SplitScan sc2 = scan_split(eh2, el, D);
    const int local = draw_split<DT, TOPP, true>(gs, eh2, el, et2, sc2, s_rem, d, k, D);
    if (local >= 0) tok = gs.e0 + local;
  }
  if (t == 0) {
    out_tokens[(size_t)b * (K + 1) + d.n] = tok;
    if (out_mass) out_mass[b] = (float)s_total;
  }
}

// A greedy request inside a sampling call (temperature 0): the residual
// tile 0 combines the argmax keys of target rows 0..K with its first wave,
// accepts drafts while each equals the top choice, and emits the top choice
// at the first mismatch (lotook.com explainer, FAQ: at temperature 0 a draft
// is accepted only if it is the target's top choice).
__device__ __forceinline__ void greedy_in_sample(const SampleArgs &a, int b) {
  const int i = threadIdx.x;  // < 64
  const int K = a.K, S = a.S;
  int am = -1, x = -1;
  bool ok = true;
  if (i <= K) {
    const size_t g0 = ((size_t)b * (K + 1) + i) * S;
    u64 best = 0;
    for (int s = 0; s < S && ok; ++s) {
      bool got = false;
      for (int it = 0; it < kSpinLimit && !got; ++it) {
        uint32_t hi, lo;
        got = ((int)unpack_u32(load_agent(&a.part_m[g0 + s]), a.epoch, &hi) &
               (int)unpack_u32(load_agent(&a.part_z[2 * (g0 + s)]), a.epoch, &lo)) != 0;
        if (got) {
          const u64 key = ((u64)hi << 32) | lo;
          best = key > best ? key : best;
        } else {
          spin_pause();
        }
      }
      ok = got;
    }
    am = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
  }
  if (i < K) x = a.tokens[(size_t)b * K + i];
  if (__ballot(!ok)) {
    if (i == 0) a.out_accepted[b] = -2;  // time-out: flag the request as failed
    return;
  }
  const uint64_t miss = __ballot(i < K && x != am);
  const int n = miss ? __builtin_ctzll(miss) : K;
  if (i <= K) a.out_tokens[(size_t)b * (K + 1) + i] = i < n ? x : (i == n ? am : -1);
  if (i < K) {
    if (a.out_p) a.out_p[(size_t)b * K + i] = 0.f;
    if (a.out_q) a.out_q[(size_t)b * K + i] = 0.f;
  }
  if (i == 0) {
    a.out_accepted[b] = n;
    if (a.out_mass) a.out_mass[b] = 0.f;
  }
}

}  // namespace

// The pointers come in as separate restrict-qualified arguments: the
// compiler may then take the uniform reads (the draft tokens above all) as
// scalar loads that do not hold up the stream's vector loads.
// MIXED: per-request parameters (temps / topps on the device); otherwise the
// batch-wide ones and no greedy requests (the per-request code stays out of
// the batch-wide kernel, where it would cost registers and issue slots).
template <int DT, bool MIXED, bool TOPP>
__global__ __launch_bounds__(kThreads) void k_sample_fused(
    const char *__restrict__ target, const char *__restrict__ draft,
    const int32_t *__restrict__ tokens, const float *__restrict__ u_accept,
    const float *__restrict__ u_sample, const float *__restrict__ temps,
    const float *__restrict__ topps, u64 *__restrict__ part_m, u64 *__restrict__ part_z,
    u64 *__restrict__ part_x, RowStat *__restrict__ rowstat, u64 *__restrict__ rtot,
    int32_t *__restrict__ out_accepted,
    int32_t *__restrict__ out_tokens, float *__restrict__ out_p, float *__restrict__ out_q,
    float *__restrict__ out_mass, SampleArgs a) {
  a.target = target;
  a.draft = draft;
  a.tokens = tokens;
  a.u_accept = u_accept;
  a.u_sample = u_sample;
  a.temps = temps;
  a.topps = topps;
  a.part_m = part_m;
  a.part_z = part_z;
  a.part_x = part_x;
  a.rowstat = rowstat;
  a.rtot = rtot;
  a.out_accepted = out_accepted;
  a.out_tokens = out_tokens;
  a.out_p = out_p;
  a.out_q = out_q;
  a.out_mass = out_mass;
  const int blk = (int)blockIdx.x;
  const int B = a.B, K = a.K, V = a.V, S = a.S, SB = a.SB;
  const int R = 2 * K + 1;
  const int nA_req = R * S;
  bool streaming;
  int b, idx;
  if (a.phase == 1) {  // streaming tiles only
    streaming = true;
    b = blk / nA_req;
    idx = blk - b * nA_req;
  } else if (a.phase == 2) {  // residual tiles only
    streaming = false;
    b = blk / SB;
    idx = blk - b * SB;
  } else {  // group g holds [streaming(g) | residual(g - lag)]
    const int lag = a.lag;
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
  ReqParams q;
  if (MIXED) {
    q = request_params(a.temps, a.topps, a.k64, a.k, a.top_p, b);
  } else {
    q.invalid = false;
    q.greedy = false;
    q.k64 = a.k64;
    q.k = a.k;
    q.top_p = a.top_p;
  }
  if (q.invalid) {  // a request's own parameters are out of range
    if (!streaming && idx == 0 && threadIdx.x <= K) {
      a.out_tokens[(size_t)b * (K + 1) + threadIdx.x] = -1;
      if (threadIdx.x == 0) a.out_accepted[b] = -3;
    }
    return;
  }
  if (streaming) {
    const int r = idx / S;
    const int s = idx - r * S;
    const int rows_t = B * (K + 1);
    const int grow = r <= K ? b * (K + 1) + r : rows_t + b * K + (r - K - 1);
    if (q.greedy) {  // top choices of the target rows; the draft rows are not read
      if (r > K) return;
      const uint64_t key = argmax_tile<DT>(row_ptr(a.target, (size_t)grow, V, DT), V, s);
      if (threadIdx.x == 0) {
        store_agent(&a.part_m[(size_t)grow * S + s], pack_u32((uint32_t)(key >> 32), a.epoch));
        store_agent(&a.part_z[2 * ((size_t)grow * S + s)], pack_u32((uint32_t)key, a.epoch));
      }
      return;
    }
    const char *rp = r <= K ? row_ptr(a.target, (size_t)grow, V, DT)
                            : row_ptr(a.draft, (size_t)(grow - rows_t), V, DT);
    // the draft token's logit, if this split holds it (for a token out of
    // range split 0 publishes -inf: probability 0, the draft is rejected).
    // Everything here is uniform across the workgroup, so it lives in scalar
    // registers: the logits are read-only for the whole call, and the aligned
    // dword holding the element (same page, so always readable) comes with a
    // scalar load through the constant address space, leaving the vector
    // queue to the stream; its bits are picked apart after the stream.  The
    // two dependent scalar loads run once the stream's loads are in flight.
    const int pos = r <= K ? r : r - K - 1;  // position; target row K has no draft token
    bool mine = false, valid = false;
    unsigned mis = 0;
    uint32_t w = 0;
    float M;
    double Z;
    uint8_t *hist = TOPP && a.part_h && q.top_p < 1.0 ? a.part_h + ((size_t)grow * S + s) * kHistBins : nullptr;
    softmax_tile<DT, TOPP>(rp, V, s, q.k, &M, &Z, [&] {
      if (r != K) {
        const int x = a.tokens[(size_t)b * K + pos];
        const int e0 = s * split_elems(DT), e1 = min(V, e0 + split_elems(DT));
        valid = x >= 0 && x < V;
        mine = (valid && x >= e0 && x < e1) || (!valid && s == 0);
        if (mine && valid) {
          typedef const __attribute__((address_space(4))) uint32_t *const_u32p;
          const uintptr_t ea = reinterpret_cast<uintptr_t>(rp) + (uintptr_t)x * elem_bytes(DT);
          mis = (unsigned)(ea & 3u);
          w = *(const_u32p)(ea - mis);
        }
      }
    }, hist, hist ? a.part_c + ((size_t)grow * S + s) * kChunksPerSplit : nullptr,
       hist ? a.part_c2 + ((size_t)grow * S + s) * kChunksPerSplit : nullptr);
    if (threadIdx.x == 0) {
      const size_t g = (size_t)grow * S + s;
      float zh, zl;
      split_f64(Z, &zh, &zl);
      store_agent(&a.part_m[g], pack_u32(__float_as_uint(M), a.epoch));
      store_agent(&a.part_z[2 * g], pack_u32(__float_as_uint(zh), a.epoch));
      store_agent(&a.part_z[2 * g + 1], pack_u32(__float_as_uint(zl), a.epoch));
      if (mine) {
        const uint32_t lx_bits = !valid ? 0xFF800000u  // -inf
                                 : DT == kBF16 ? (mis ? (w & 0xFFFF0000u) : (w << 16)) : w;
        store_agent(a.part_x + ((size_t)b * K + pos) * 2 + (r <= K ? 0 : 1),
                    pack_u32(lx_bits, a.epoch));
      }
    }
    return;
  }
  if (q.greedy) {
    if (idx == 0 && threadIdx.x < 64) greedy_in_sample(a, b);
    return;
  }
  __shared__ ResidLds rl;
  if (a.rowstat)
    residual_tile<DT, true>(a.target, a.draft, a.tokens, a.u_accept, a.u_sample, B, K, V, S, SB,
                            q.k64, q.k, a.epoch, a.part_m, a.part_z, a.part_x, a.rowstat,
                            a.rtot, a.out_accepted, a.out_tokens, a.out_p, a.out_q,
                            a.out_mass, b, idx, rl);
  else
    residual_tile<DT, false>(a.target, a.draft, a.tokens, a.u_accept, a.u_sample, B, K, V, S,
                             SB, q.k64, q.k, a.epoch, a.part_m, a.part_z, a.part_x, a.rowstat,
                             a.rtot, a.out_accepted, a.out_tokens, a.out_p, a.out_q,
                             a.out_mass, b, idx, rl);
}

// The ratio tests of a top-p call with batch-wide parameters, one workgroup
// per request, between the nucleus launches and the residual tiles: the
// outcome, the emitted drafts and the per-position probabilities are
// written here once, and the residual tiles read the request's Decision
// instead of each deciding again.
__global__ __launch_bounds__(kThreads) void k_topp_decide(SampleArgs a) {
  __shared__ DecideLds lds;
  __shared__ Decision sdec;
  __shared__ int s_ok;
  const int b = (int)blockIdx.x;
  if (!decide(a.tokens, a.u_accept, a.B, a.K, a.S, a.k64, a.k, a.part_m, a.part_z, a.part_x,
              a.epoch, a.rowstat, b, true, a.out_accepted, a.out_tokens, a.out_p, a.out_q, lds,
              &sdec, &s_ok)) {
    if (threadIdx.x == 0) {
      a.out_accepted[b] = -2;  // time-out: flag the request as failed
      Decision d = {};
      d.n = -1;
      a.dec[b] = d;
    }
    return;
  }
  if (threadIdx.x == 0) a.dec[b] = sdec;
}

hipError_t launch_topp_decide(const SampleArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(k_topp_decide, dim3(a.B), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// After the decide launch of a top-p call: the residual (or bonus) mass of
// every residual split of each request's drawn row pair, one workgroup per
// (request, split), stored as a plain fp64 value for the draw launch.  No
// workgroup waits for another: the launch streams at the memory's pace.
constexpr int kMassSplits = 2;  // residual splits per workgroup of the mass launch

// Whether this lane's body groups of a residual split can hold an element of
// the target row's nucleus (logit >= tau): p' is 0 below tau, and so is the
// residual max(0, p' - q').  The lane's kVecPerThreadB groups lie in one
// 128-byte line of a streaming split (residual and streaming splits start
// at multiples of 16 KB, so both share the row's 16-byte phase, and lines are
// aligned runs of eight groups); the streaming pass recorded that line's
// maximum in part_c (entry g * 8 + u for the groups 8 g .. 8 g
// + 7 of slot u, i.e. body groups u kThreads + 8 g .. + 7).  Groups that no
// recorded line covers (a streaming split's scalar tail and head) are always
// loaded.
template <int DT>
__device__ __forceinline__ bool lane_in_nucleus(const SplitGeo &g, const char *rt, int V,
                                                const uint32_t *cm_row, float tau) {
  constexpr int EPV = 16 / elem_bytes(DT);
  constexpr int VB = kVecPerThreadB;
  static_assert(8 % VB == 0 && kChunkLanes == 8, "a lane's groups lie in one line");
  const int v0 = threadIdx.x * VB;
  if (v0 >= g.nvec) return false;  // past the body: never counted
  const int e = g.e0 + g.head + v0 * EPV;  // the row element that starts the lane's groups
  const int s = e / split_elems(DT);
  const Span sp = split_span(rt, V, s, DT);
  const int off = e - sp.e0 - sp.head;
  if (off < 0 || off % EPV != 0) return true;
  const int vb = off / EPV;
  if (vb % VB != 0 || vb + VB > sp.nvec) return true;
  const int entry = ((vb % kThreads) / kChunkLanes) * kChunkLanes + vb / kThreads;
  return !(__uint_as_float(cm_row[(size_t)s * kChunksPerSplit + entry]) < tau);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_resid_mass(SampleArgs a) {
  __shared__ double red[kThreads / 64];
  __shared__ double eh[kMassSplits], et[kMassSplits];
  const int per_req = (a.SB + kMassSplits - 1) / kMassSplits;
  const int b = (int)blockIdx.x / per_req;
  const int s0 = ((int)blockIdx.x - b * per_req) * kMassSplits;
  const Decision d = a.dec[b];
  if (d.n < 0) return;
  const size_t trow = (size_t)b * (a.K + 1) + d.n;
  const char *rt = row_ptr(a.target, trow, a.V, DT);
  const char *rd = d.mode == kModeResidual ? row_ptr(a.draft, (size_t)b * a.K + d.n, a.V, DT) : rt;
  // only lines of the target row that can reach its nucleus are read (both
  // rows); the rest holds no residual mass.  Every split's loads issued
  // before any is used.
  const uint32_t *cm_row = a.part_c ? a.part_c + trow * a.S * kChunksPerSplit : nullptr;
  const bool skip = cm_row && d.tau_t > -INFINITY;
  SplitGeo g[kMassSplits];
  bool need[kMassSplits];
#pragma unroll
  for (int j = 0; j < kMassSplits; ++j) {
    g[j] = split_geo<DT>(rt, rd, a.V, min(s0 + j, a.SB - 1));
    need[j] = !skip || !g[j].aligned || lane_in_nucleus<DT>(g[j], rt, a.V, cm_row, d.tau_t);
  }
  LaneGroups mine[kMassSplits];
#pragma unroll
  for (int j = 0; j < kMassSplits; ++j) {
    if (need[j]) {
      load_lane<DT, false>(g[j], mine[j]);
    } else {
#pragma unroll
      for (int u = 0; u < kVecPerThreadB; ++u) mine[j].wt[u] = mine[j].wq[u] = neg_inf_vec<DT>();
    }
  }
  if (threadIdx.x < kMassSplits && s0 + (int)threadIdx.x < a.SB) {
    const int j = threadIdx.x;
    const SplitGeo gj = split_geo<DT>(rt, rd, a.V, s0 + j);
    eh[j] = range_mass<DT, true, false>(gj, 0, gj.head, d, a.k);
    et[j] = range_mass<DT, true, false>(gj, gj.tail0, gj.n, d, a.k);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kMassSplits; ++j) {
    if (s0 + j >= a.SB) break;
    const double lm = lane_mass<DT, true, false>(g[j], mine[j], d, a.k);
    const double tot = block_sum(lm + (threadIdx.x == 0 ? eh[j] + et[j] : 0.0), red);
    if (threadIdx.x == 0)
      reinterpret_cast<double *>(a.rtot)[(size_t)b * a.SB + s0 + j] = tot;
  }
}

// The draw of a top-p call, one workgroup per request: the split where the
// cumulative residual mass passes u * S (from the split masses of the mass
// launch), then that split of the row pair read again and scanned; if the
// residual mass is not above the resolution level, the draw from p' instead
// (every split's p' mass, then the same steps).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_resid_draw(SampleArgs a) {
  __shared__ DrawLds D;
  __shared__ double red[kThreads / 64];
  __shared__ int s_split;
  __shared__ double s_rem, s_total;
  const int t = threadIdx.x, b = (int)blockIdx.x, SB = a.SB, K = a.K;
  const Decision d = a.dec[b];
  if (d.n < 0) return;
  const char *rt = row_ptr(a.target, (size_t)b * (K + 1) + d.n, a.V, DT);
  const char *rd = d.mode == kModeResidual ? row_ptr(a.draft, (size_t)b * K + d.n, a.V, DT) : rt;
  const float us = a.u_sample[b];
  const double *tot = reinterpret_cast<const double *>(a.rtot) + (size_t)b * SB;
  for (int i = t; i < SB; i += kThreads) D.tot[i] = tot[i];
  __syncthreads();
  if (SB <= 64) {
    if (t < 64) {
      double rem, total;
      const int split = pick_split_wave(t < SB ? D.tot[t] : 0.0, SB, us, &rem, &total);
      if (t == 0) {
        s_split = split;
        s_rem = rem;
        s_total = total;
      }
    }
  } else if (t == 0) {
    double rem, total;
    s_split = pick_split(D.tot, SB, us, &rem, &total);
    s_rem = rem;
    s_total = total;
  }
  __syncthreads();
  const bool use_p = !(s_total > kResidualResolution);
  if (use_p) {  // S = 0 in exact arithmetic: p' of every split, then the pick again
    for (int i = 0; i < SB; ++i) {
      const SplitGeo gi = split_geo<DT>(rt, rd, a.V, i);
      LaneGroups li;
      load_lane<DT, true>(gi, li);
      double v = lane_mass<DT, true, true>(gi, li, d, a.k);
      if (t == 0)
        v += range_mass<DT, true, true>(gi, 0, gi.head, d, a.k) +
             range_mass<DT, true, true>(gi, gi.tail0, gi.n, d, a.k);
      v = block_sum(v, red);
      if (t == 0) D.tot[i] = v;
    }
    __syncthreads();
    if (t == 0) {
      double rem, total;
      s_split = pick_split(D.tot, SB, us, &rem, &total);
      s_rem = rem;
      s_total = total;
    }
    __syncthreads();
  }
  int tok = -1;
  const int split = s_split;
  if (split >= 0) {
    const SplitGeo g = split_geo<DT>(rt, rd, a.V, split);
    LaneGroups mine;
    if (use_p) load_lane<DT, true>(g, mine);
    else load_lane<DT, false>(g, mine);
    const double el = use_p ? lane_mass<DT, true, true>(g, mine, d, a.k)
                            : lane_mass<DT, true, false>(g, mine, d, a.k);
    if (t == 0) {
      D.eh = use_p ? range_mass<DT, true, true>(g, 0, g.head, d, a.k)
                   : range_mass<DT, true, false>(g, 0, g.head, d, a.k);
      D.et = use_p ? range_mass<DT, true, true>(g, g.tail0, g.n, d, a.k)
                   : range_mass<DT, true, false>(g, g.tail0, g.n, d, a.k);
    }
    __syncthreads();
    const double eh = D.eh, et = D.et;
    const SplitScan sc = scan_split(eh, el, D);
    const int local = use_p ? draw_split<DT, true, true>(g, eh, el, et, sc, s_rem, d, a.k, D)
                            : draw_split<DT, true, false>(g, eh, el, et, sc, s_rem, d, a.k, D);
    if (local >= 0) tok = g.e0 + local;
  }
  if (t == 0) {
    a.out_tokens[(size_t)b * (K + 1) + d.n] = tok;
    if (a.out_mass) a.out_mass[b] = (float)s_total;
  }
}

hipError_t launch_topp_residual(const SampleArgs &a, int dtype, hipStream_t stream) {
  if (dtype == kBF16) {
    hipLaunchKernelGGL(k_resid_mass<kBF16>, dim3(a.B * ((a.SB + kMassSplits - 1) / kMassSplits)),
                       dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(k_resid_draw<kBF16>, dim3(a.B), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(k_resid_mass<kF32>, dim3(a.B * ((a.SB + kMassSplits - 1) / kMassSplits)),
                       dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(k_resid_draw<kF32>, dim3(a.B), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_sample(const SampleArgs &args, int dtype, hipStream_t stream) {
  SampleArgs a = args;
  const int nA = a.B * (2 * a.K + 1) * a.S;
  const int nB = a.B * a.SB;
  // phase: 0 = whole call, 1 = streaming tiles only, 2 = residual tiles only
  const int blocks = a.phase == 0 ? nA + nB : a.phase == 1 ? nA : nB;
  a.lag = std::max(1, std::min(a.lag, a.B));
  const bool mixed = a.temps != nullptr || a.topps != nullptr;
  // the streaming tiles of a top-p call also count and record chunk maxima
  const bool topp = a.part_h != nullptr && a.phase == 1;
  auto kern = dtype == kBF16
                  ? (mixed ? (topp ? k_sample_fused<kBF16, true, true> : k_sample_fused<kBF16, true, false>)
                           : (topp ? k_sample_fused<kBF16, false, true> : k_sample_fused<kBF16, false, false>))
                  : (mixed ? (topp ? k_sample_fused<kF32, true, true> : k_sample_fused<kF32, true, false>)
                           : (topp ? k_sample_fused<kF32, false, true> : k_sample_fused<kF32, false, false>));
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), 0, stream, a.target, a.draft, a.tokens,
                     a.u_accept, a.u_sample, a.temps, a.topps, a.part_m, a.part_z, a.part_x,
                     a.rowstat, a.rtot, a.out_accepted, a.out_tokens, a.out_p, a.out_q,
                     a.out_mass, a);
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
    const void *fn = d ? (const void *)k_sample_fused<kBF16, false, false>
                       : (const void *)k_sample_fused<kF32, false, false>;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess)
      per_cu = 4;
    cache[d] = std::max(1, cus * per_cu);
  }
  return cache[d];
}

}  // namespace sv
