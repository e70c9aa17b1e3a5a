// Shared host/device constants, workspace records and the workspace layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <math.h>

namespace sv {

typedef unsigned long long u64;

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// Streaming geometry: a workgroup of 256 lanes streams one split of one row,
// each lane holding 8 16-byte loads in flight (32 KB per workgroup).
constexpr int kThreads = 256;
constexpr int kVecPerThread = 8;

__host__ __device__ constexpr int elem_bytes(int dtype) { return dtype == kBF16 ? 2 : 4; }
__host__ __device__ constexpr int split_elems(int dtype) {
  return kThreads * kVecPerThread * (16 / elem_bytes(dtype));
}
__host__ __device__ inline int num_splits(int V, int dtype) {
  return (V + split_elems(dtype) - 1) / split_elems(dtype);
}

// Residual pass geometry: splits of 4 vectors per lane, so that the draw for
// one request is spread over several workgroups.
constexpr int kVecPerThreadB = 4;
__host__ __device__ constexpr int split_elems_b(int dtype) {
  return kThreads * kVecPerThreadB * (16 / elem_bytes(dtype));
}
__host__ __device__ inline int num_splits_b(int V, int dtype) {
  return (V + split_elems_b(dtype) - 1) / split_elems_b(dtype);
}

// k = log2(e) / T as an unevaluated sum hi + lo of two floats, lo > 0.
struct Scale {
  float hi, lo;
};

// k = log2(e) / T split into float hi + lo with lo > 0 (lo carries the
// rounding of hi, so the product (l - m) * k keeps ~1 ulp accuracy per
// element).  The same steps on the host and on the device.
__host__ __device__ inline Scale make_scale(double k64) {
  float hi = (float)k64;
  if ((double)hi >= k64) hi = nextafterf(hi, 0.0f);
  float lo = (float)(k64 - (double)hi);
  if (!(lo > 0.0f)) {
    hi = nextafterf(hi, 0.0f);
    lo = (float)(k64 - (double)hi);
  }
  return Scale{hi, lo};
}
constexpr double kLog2e = 1.4426950408889634;

// One row's softmax statistics after combining its splits (and top-p).
struct RowStat {
  double z;   // sum over the row of 2^((l - m) k)
  double zk;  // kept (nucleus) mass in the same units; == z without top-p
  float m;    // row maximum
  float tau;  // smallest kept logit; -inf keeps everything
};

// Per request: the outcome of the ratio tests and what the residual draw
// needs.  A token's mass in row n is 2^((l - m) k) / kept mass, with the
// difference l - m exact, so that equal rows give equal masses bit for bit
// and a row's maximum weighs exactly 1 / kept mass.
struct Decision {
  int n;                // accepted drafts (0..K)
  int mode;             // kModeResidual or kModeBonus
  float m_t, m_d;       // maxima of target row n / draft row n
  float tau_t, tau_d;   // smallest kept logits (-inf: all kept)
  // 1 / kept mass (the mass is at least 1) as an unevaluated fp32 pair hi + lo:
  // one rounding of each inverse to fp32 would scale every p' (and every q')
  // by its own factor within 2^-24 of 1, a shift that max(0, p' - q') does
  // not cancel and that S magnifies when it is small; inv_d = 0 for the
  // bonus draw (r = p')
  float inv_t, inv_t_lo, inv_d, inv_d_lo;
};
constexpr int kModeResidual = 0;
constexpr int kModeBonus = 1;

// Largest number of residual splits per row (the draw stages them in LDS).
constexpr int kMaxSplitsB = 512;

// A residual mass S = sum max(0, p' - q') at or below 2^-20 of the unit mass
// is taken as empty and the replacement is drawn from p' instead: S = 0 is
// impossible after a rejection in exact arithmetic, and at this level (twice
// the total rounding of p' and q' as float32 values, e.g. two equal rows
// whose normalisers were summed in different orders) the residual holds
// rounding alone.
constexpr double kResidualResolution = 9.5367431640625e-07;

// Top-p: a streaming tile also counts its split's elements by distance from
// the split maximum on the grid floor(l * k * kHistPerLog2) (1/64 log2 unit,
// k = log2(e) / T), bins 0 .. kHistBins-1 (24 log2 units), 8-bit counts
// that stop at kCountSat (a saturated bin sends its row to the fallback).
constexpr int kHistBins = 1536;
constexpr float kHistPerLog2 = 64.f;
constexpr unsigned kCountSat = 255u;
// Top-p: keys of a row's band kept for the cut (more: the cut reads the row).
constexpr int kBandKeys = 4096;
// Top-p: a streaming tile also records, per chunk, the chunk's maximum
// exactly (its fp32 pattern) and a bound on its second largest element (the
// upper half of that element's fp32 pattern, rounded so the value it denotes
// is not below the element), a chunk being one vector slot u of a group g of
// eight consecutive lanes (8 x 16 bytes: one 128-byte line).  Entry g *
// kVecPerThread + u: lane t writes entry t, and a lane reads its slots'
// entries in one load.
constexpr int kChunkLanes = 8;
constexpr int kChunksPerSplit = kThreads * kVecPerThread / kChunkLanes;
static_assert(kChunkLanes == kVecPerThread, "lane t writes entry t");

// Top-p, per row, from the band kernel to the gather and cut kernels.
struct TopBand {
  double z;       // sum over the row of 2^((l - m) k)
  float m;        // row maximum
  int state;      // kTopDone (RowStat written), kTopCounts (band valid), kTopFallback
  int blo, bhi;   // the band of count bins that holds the cut
};
constexpr int kTopDone = 0;
constexpr int kTopCounts = 1;
constexpr int kTopFallback = 2;

// Arguments of the fused sampling kernel (and what a call shares with the
// top-p kernel).  temps / topps: per-request temperature and top-p on the
// device (NULL: the batch-wide k, k64, top_p apply).
struct SampleArgs {
  const char *target, *draft;
  const int32_t *tokens;
  const float *u_accept, *u_sample;
  const float *temps, *topps;
  int B, K, V, S, SB;
  double k64, top_p;
  Scale k;
  u64 epoch;
  int phase, lag;
  u64 *part_m, *part_z, *part_x;
  RowStat *rowstat;
  u64 *rtot;  // per (request, residual split): the split's mass as two tagged fp32 words
  uint8_t *part_h;  // top-p: per (row, split) kHistBins element counts (null otherwise)
  uint32_t *part_c;   // top-p: per (row, split) kChunksPerSplit chunk maxima (fp32 patterns)
  uint16_t *part_c2;  // top-p: per (row, split) kChunksPerSplit bounds on the chunks' second largest elements
  TopBand *topband;  // top-p: per row
  unsigned *band_n;  // top-p: per row, keys in the band (the list holds the first kBandKeys)
  uint32_t *band_keys;  // top-p: per row, kBandKeys keys
  double *band_above;   // top-p: per row, exact mass above the band
  Decision *dec;        // top-p, batch-wide parameters: per request, the outcome of the
                        // ratio tests, decided once before the residual tiles (n = -1:
                        // the request failed)
  int32_t *out_accepted, *out_tokens;
  float *out_p, *out_q, *out_mass;
};

// A request's sampling parameters, as the kernels see them.
struct ReqParams {
  bool invalid;  // temperature not finite or < 0, or top_p not in (0, 1]
  bool greedy;   // temperature 0
  double k64, top_p;
  Scale k;
};

__host__ __device__ inline ReqParams request_params(const float *temps, const float *topps,
                                                    double k64, Scale k, double top_p, int b) {
  ReqParams q;
  q.invalid = false;
  q.greedy = false;
  q.k64 = k64;
  q.k = k;
  q.top_p = top_p;
  if (temps) {
    const float T = temps[b];
    if (!(T >= 0.0f) || !(T < INFINITY)) {
      q.invalid = true;
    } else if (T == 0.0f) {
      q.greedy = true;
    } else {
      q.k64 = kLog2e / (double)T;
      if (!(q.k64 <= 3.0e38)) q.invalid = true;
      else q.k = make_scale(q.k64);
    }
  }
  if (topps) {
    const float p = topps[b];
    if (!(p > 0.0f) || !(p <= 1.0f)) q.invalid = true;
    else q.top_p = (double)p;
  }
  return q;
}

struct Layout {
  int S = 0;       // streaming splits per row
  int SB = 0;      // residual splits per row (sampling)
  int rows = 0;    // logit rows streamed
  size_t part_m = 0, part_z = 0, part_x = 0, part_key = 0, part_tag = 0, rowstat = 0;
  size_t rtot = 0, part_h = 0, part_c = 0, part_c2 = 0, topband = 0, band_n = 0, band_keys = 0,
         band_above = 0;
  size_t dec = 0;
  // sampling: part_m one self-validating u64 word per (row, split) (the split
  // maximum), part_z two (the split mass as fp32 hi + lo);
  // part_x one word per (request, position, target / draft): the logit of the
  // draft token, written by the streaming tile whose split holds it
  size_t total = 0;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// op: 0 greedy, 1 sample, 2 tree.  KN = K (greedy/sample) or N (tree).
inline Layout make_layout(int op, int B, int KN, int V, int dtype, int use_top_p) {
  Layout L;
  L.S = num_splits(V, dtype);
  if (op == 1)
    L.rows = B * (2 * KN + 1);
  else if (op == 0)
    L.rows = B * (KN + 1);
  else
    L.rows = B * KN;
  size_t cells = (size_t)L.rows * (size_t)L.S;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  if (op == 1) {
    L.SB = num_splits_b(V, dtype);
    L.part_m = take(cells * sizeof(u64));
    L.part_z = take(cells * 2 * sizeof(u64));
    L.part_x = take((size_t)B * (size_t)KN * 2 * sizeof(u64));
    L.rowstat = use_top_p ? take((size_t)L.rows * sizeof(RowStat)) : 0;
    L.rtot = take((size_t)B * (size_t)L.SB * 2 * sizeof(u64));
    if (use_top_p) {
      L.part_h = take(cells * kHistBins * sizeof(uint8_t));
      L.part_c = take(cells * kChunksPerSplit * sizeof(uint32_t));
      L.part_c2 = take(cells * kChunksPerSplit * sizeof(uint16_t));
      L.topband = take((size_t)L.rows * sizeof(TopBand));
      L.band_n = take((size_t)L.rows * sizeof(unsigned));
      L.band_keys = take((size_t)L.rows * kBandKeys * sizeof(uint32_t));
      L.band_above = take((size_t)L.rows * sizeof(double));
      L.dec = take((size_t)B * sizeof(Decision));
    }
  } else {
    L.part_key = take(cells * sizeof(uint64_t));
    L.part_tag = take(cells * sizeof(u64));
  }
  L.total = off;
  return L;
}

}  // namespace sv
