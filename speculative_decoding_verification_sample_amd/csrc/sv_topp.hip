// Top-p (nucleus) threshold per logit row, exact, without a sort.
//
// After temperature, keep the largest logits, whole tie groups, until their
// mass first reaches top_p of the row, and renormalise (ariser.io review,
// section "같은 분포를 지키는 작은 장치": temperature / top-p must be applied
// to both p and q before the test; the nucleus rule itself is the plainest
// reading, the pages name it only).  The streaming pass has left each
// row's maximum M, normaliser Z and, per split, counts of its elements by
// distance from the maximum on a shared grid (bins of 1/64 log2 unit).
// Three launches:
//   band (one workgroup per row): merge the counts; an element of bin J
//     weighs between 2^-(J+phi)/64 and 2^-(J+phi-1)/64, so running bounds
//     of the mass from the top pin the element where the cumulative mass
//     reaches top_p * Z to a band of bins [b_lo, b_hi] (bins are value
//     intervals: tie groups never split).  The counts cover 24 log2 units;
//     the elements beyond weigh so little that all of them together stay
//     under half of the mass top_p leaves out, so the cut lies inside.
//   gather (one workgroup per row): the exact mass of the row's elements
//     nearer than the band, and the band's elements as order-preserving
//     value keys in a per-row list; the streaming pass's record of each
//     128-byte line (its maximum, exactly, and a bound on its second
//     element) gives the lines with one such element without a read, and
//     only the lines with two or more are read.
//   cut (one workgroup per row): radix rounds of 8 bits over the keys,
//     accumulating mass from the top, until one distinct value remains:
//     that value is tau, the mass at or above it is the kept mass.
// A row the counts cannot cover (a small normaliser, a huge logit scale)
// takes the fallback in the cut launch: an fp64 LDS histogram of tempered
// mass over bins of the distance (M - l) * log2(e)/T, 1/8 log2 unit wide,
// finds the bin where the cumulative mass reaches top_p * Z, one more pass
// gathers that bin, and the same radix rounds finish.
#include "sv_device.hpp"
#include "sv_kernels.hpp"
#include "sv_tiles.hpp"

namespace sv {

constexpr int kTopThreads = 512;
constexpr int kTopWaves = kTopThreads / 64;
constexpr int kBins = 256;
constexpr float kBinsPerLog2 = 8.f;
constexpr int kCand = 4096;  // keys of the selected bin or band held in LDS
constexpr int kMergeSplits = 20;  // splits' counts staged in LDS at a time (30 KB)
// Slack on the count bounds: covers the fp32 rounding of grid positions
// (|M kk| < 2^18: under 0.03 of a bin, a factor 3.4e-4) and of the masses;
// a wider slack only widens the band.
constexpr double kBoundSlack = 1e-3;

namespace {

__device__ __forceinline__ int dist_bin(float x, float M, float kr) {
  const float d = (M - x) * kr;   // >= 0; +inf for x = -inf
  return d < (float)(kBins - 1) ? (int)d : kBins - 1;
}

// Bin of x on the counting grid, relative to the row maximum's cell F =
// floor(M kk) (the streaming tiles' grid); kHistBins for -inf or beyond.
__device__ __forceinline__ int grid_bin(float x, float F, float kk) {
  if (!(x > -INFINITY)) return kHistBins;
  const float j = F - floorf(x * kk);
  return j < (float)kHistBins ? (int)j : kHistBins;
}

// Calls f(j, x) for every element of a row: 16-byte vector body, scalar
// head / tail, four vectors in flight per lane.
template <int DT, class F>
__device__ __forceinline__ void for_row(const char *row, int V, F &&f) {
  constexpr int ES = elem_bytes(DT);
  constexpr int EPV = 16 / ES;
  const int t = threadIdx.x;
  const uintptr_t a = reinterpret_cast<uintptr_t>(row);
  const int head = min(V, (int)(((16u - (unsigned)(a & 15u)) & 15u) / ES));
  const int nvec = (V - head) / EPV;
  const int tail = V - head - nvec * EPV;
  if (t < head) f(t, load_elem(row, t, DT));
  const u32x4 *body = reinterpret_cast<const u32x4 *>(row + (size_t)head * ES);
  for (int v0 = 0; v0 < nvec; v0 += 4 * kTopThreads) {
    u32x4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * kTopThreads + t;
      if (v < nvec) w[u] = body[v];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * kTopThreads + t;
      if (v < nvec) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) f(head + v * EPV + e, vec_elem(w[u], e, DT));
      }
    }
  }
  if (t < tail) {
    const int j = head + nvec * EPV + t;
    f(j, load_elem(row, j, DT));
  }
}


// The row's place in the call and its request's sampling parameters.
struct TopRow {
  const char *rp;
  ReqParams q;
};
template <int DT>
__device__ __forceinline__ TopRow top_row(const SampleArgs &a, int row) {
  const int rows_t = a.B * (a.K + 1);
  const size_t row_bytes = (size_t)a.V * elem_bytes(DT);
  TopRow r;
  r.rp = row < rows_t ? a.target + (size_t)row * row_bytes
                      : a.draft + (size_t)(row - rows_t) * row_bytes;
  const int b = row < rows_t ? row / (a.K + 1) : (row - rows_t) / a.K;
  r.q = request_params(a.temps, a.topps, a.k64, a.k, a.top_p, b);
  return r;
}

}  // namespace

// ---------------------------------------------------------------------------
// band: per row, M and Z from the streaming partials, then the counts
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kTopThreads) void k_topp_band(SampleArgs a) {
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int V = a.V, S = a.S;
  const TopRow tr = top_row<DT>(a, row);
  if (tr.q.invalid || tr.q.greedy) {  // no softmax statistics for this request
    if (t == 0) {
      TopBand tb;
      tb.z = 0.0;
      tb.m = -INFINITY;
      tb.state = kTopDone;
      tb.blo = tb.bhi = 0;
      a.topband[row] = tb;
    }
    return;
  }
  const Scale k = tr.q.k;
  const double k64 = tr.q.k64, top_p = tr.q.top_p;
  const u64 *pm = a.part_m + (size_t)row * S;
  const u64 *pz = a.part_z + (size_t)row * S * 2;
  const float kk = (k.hi + k.lo) * kHistPerLog2;

  __shared__ unsigned cntf[kHistBins];
  __shared__ double wsum[2][kTopWaves];
  __shared__ float sM;
  __shared__ double sZ, s_fu, s_fl;
  __shared__ int s_fast, s_wbl[kTopWaves], s_wbh[kTopWaves];

  if (t < 64) {  // the streaming kernel has completed: every partial is in place
    float M = -INFINITY;
    for (int s = t; s < S; s += 64) M = fmaxf(M, payload_f32(pm[s]));
    M = wave_max(M);
    M = __shfl(M, 63, 64);
    double Z = 0.0;
    for (int s = t; s < S; s += 64) {
      const float m = payload_f32(pm[s]);
      const double z = (double)payload_f32(pz[2 * s]) + (double)payload_f32(pz[2 * s + 1]);
      if (m > -INFINITY) Z += z * exp2(((double)m - (double)M) * k64);
    }
    Z = wave_sum(Z);
    if (t == 63) {
      sM = M;
      sZ = Z;
      // the counts cover the cut when the elements beyond them (each at
      // most 2^-(kHistBins-1)/64) weigh less than half of (1 - top_p) Z,
      // and the grid positions are accurate to a small part of a bin
      s_fast = M > -INFINITY && fabsf(M * kk) < 262144.f && top_p < 1.0 &&
               (double)V * exp2(-(double)(kHistBins - 1) / kHistPerLog2) <= 0.5 * (1.0 - top_p) * Z;
      // the row's factors of the count bounds below: an element of bin J
      // weighs between 2^-(J+phi)/64 and 2^-(J+phi-1)/64, phi = M kk -
      // floor(M kk) (fp64 exponentials, once per row)
      const float phi = M * kk - floorf(M * kk);
      s_fu = exp2((double)(1.f - phi) / kHistPerLog2);
      s_fl = exp2(-(double)phi / kHistPerLog2);
    }
  }
  __syncthreads();
  const float M = sM;
  const double Z = sZ;
  if (!(top_p < 1.0)) {  // no nucleus for this request: everything is kept
    if (t == 0) {
      RowStat rs;
      rs.m = M;
      rs.z = Z;
      rs.tau = -INFINITY;
      rs.zk = Z;
      a.rowstat[row] = rs;
      TopBand tb;
      tb.z = Z;
      tb.m = M;
      tb.state = kTopDone;
      tb.blo = tb.bhi = 0;
      a.topband[row] = tb;
    }
    return;
  }
  if (!s_fast) {
    if (t == 0) {
      TopBand tb;
      tb.z = Z;
      tb.m = M;
      tb.state = kTopFallback;
      tb.blo = tb.bhi = 0;
      a.topband[row] = tb;
    }
    return;
  }
  const double goal = top_p * Z;
  const float F = floorf(M * kk);

  // merge the splits' counts: split s's bin j is the row's bin j + off_s,
  // off_s = floor(M kk) - floor(m_s kk) >= 0.  Up to kMergeSplits splits at
  // a time are staged in LDS by 16-byte loads, each split's counts behind a
  // guard of zero words.  Thread t < kHistBins / 4 sums row bins 4t .. 4t+3:
  // the four bytes at 4t - off_s of each staged split (one byte-align of the
  // two words that hold them; bytes before the split's first bin come from
  // its guard) are spread into two 16-bit lanes per word, even bins and odd
  // bins, so that one add counts two bins (a group adds at most
  // kMergeSplits * 255 per lane: no carries).  A saturated count (some bin
  // of a split holds more than kCountSat elements) leaves the row to the
  // fallback.
  constexpr int kGuardW = 4;                          // 16 bytes: rows stay 16-byte aligned
  constexpr int kRowW = kGuardW + kHistBins / 4 + 4;  // guard, counts, pad
  __shared__ uint32_t stage[kMergeSplits][kRowW];
  __shared__ int s_off[kMergeSplits];
  __shared__ int s_sat;
  if (t == 0) s_sat = 0;
  for (int i = t; i < kMergeSplits * 8; i += kTopThreads) {  // guards and pads
    const int sp = i >> 3, q = i & 7;
    stage[sp][q < 4 ? q : kRowW - 8 + q] = 0u;
  }
  constexpr int kChunks = kHistBins / 16;  // 16-byte items per split
  constexpr int kPer = kHistBins / kTopThreads;  // row bins per thread in the bounds below
  constexpr int kStageIt = (kMergeSplits * kChunks + kTopThreads - 1) / kTopThreads;
  const uint8_t *h0 = a.part_h + (size_t)row * S * kHistBins;
  const bool merger = t < kHistBins / 4;
  unsigned acc[4] = {0u, 0u, 0u, 0u};
  bool sat = false;
  for (int g0 = 0; g0 < S; g0 += kMergeSplits) {
    const int gs = min(kMergeSplits, S - g0), items = gs * kChunks;
    u32x4 v[kStageIt];
#pragma unroll
    for (int u = 0; u < kStageIt; ++u) {
      const int i = t + u * kTopThreads;
      if (i < items) v[u] = reinterpret_cast<const u32x4 *>(h0 + (size_t)g0 * kHistBins)[i];
    }
    if (t < gs) {
      const float ms = payload_f32(pm[g0 + t]);
      s_off[t] = ms > -INFINITY ? (int)(F - floorf(ms * kk)) : -1;  // -1: an empty split
    }
#pragma unroll
    for (int u = 0; u < kStageIt; ++u) {
      const int i = t + u * kTopThreads;
      if (i < items) {
        const int sp = i / kChunks, c = i - sp * kChunks;
        *reinterpret_cast<u32x4 *>(&stage[sp][kGuardW + 4 * c]) = v[u];
#pragma unroll
        for (int q = 0; q < 4; ++q)  // a byte 0xFF: a zero byte of ~w
          sat |= ((~v[u][q] - 0x01010101u) & v[u][q] & 0x80808080u) != 0u;
      }
    }
    __syncthreads();
    if (merger) {
      uint32_t ev = 0u, od = 0u;  // 16-bit lanes: bins 4t, 4t+2 / 4t+1, 4t+3
      for (int sp = 0; sp < gs; ++sp) {
        const int off = s_off[sp];
        const int o = 4 * t - off;  // the byte of row bin 4t in split sp
        if (off < 0 || o <= -4) continue;
        const int b = o + 4 * kGuardW;
        const uint32_t x = __builtin_amdgcn_alignbyte(stage[sp][(b >> 2) + 1], stage[sp][b >> 2],
                                                      (uint32_t)(b & 3));
        ev += x & 0x00FF00FFu;
        od += (x >> 8) & 0x00FF00FFu;
      }
      acc[0] += ev & 0xFFFFu;
      acc[1] += od & 0xFFFFu;
      acc[2] += ev >> 16;
      acc[3] += od >> 16;
    }
    __syncthreads();
  }
  if (merger) {
#pragma unroll
    for (int e = 0; e < 4; ++e) cntf[4 * t + e] = acc[e];
  }
  if (sat) s_sat = 1;
  __syncthreads();
  // running upper / lower bounds of the mass from the top: b_lo = the first
  // bin where the upper bound reaches the goal, b_hi = the first where the
  // lower bound does
  {
    // bin J's bounds: 2^-J/64 (one fp32 exponential per bin) times the
    // row's two factors
    const double fu = s_fu, fl = s_fl;
    double up[kPer], lo[kPer], su = 0.0, sl = 0.0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int bb = t * kPer + j;
      const double c = (double)cntf[bb] * (double)exp2f((float)bb * (-1.f / kHistPerLog2));
      up[j] = c * fu;
      lo[j] = c * fl;
      su += up[j];
      sl += lo[j];
    }
    const double iu = wave_incl_scan(su), il = wave_incl_scan(sl);
    if ((t & 63) == 63) {
      wsum[0][w] = iu;
      wsum[1][w] = il;
    }
    __syncthreads();
    double cu = iu - su, cl = il - sl;
#pragma unroll
    for (int u = 0; u < kTopWaves; ++u) {
      if (u < w) {
        cu += wsum[0][u];
        cl += wsum[1][u];
      }
    }
    int bl = kHistBins, bh = kHistBins;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      cu += up[j];
      cl += lo[j];
      if (bl == kHistBins && cu * (1.0 + kBoundSlack) >= goal) bl = t * kPer + j;
      if (bh == kHistBins && cl * (1.0 - kBoundSlack) >= goal) bh = t * kPer + j;
    }
    // thread t holds bins kPer t .. kPer t + kPer - 1, so the first bins
    // are those of the lowest lane (of the lowest wave) that has them
    const uint64_t hl = __ballot(bl < kHistBins), hh = __ballot(bh < kHistBins);
    const int wl = hl ? __builtin_amdgcn_readlane(bl, (int)__builtin_ctzll(hl)) : kHistBins;
    const int wh = hh ? __builtin_amdgcn_readlane(bh, (int)__builtin_ctzll(hh)) : kHistBins;
    if ((t & 63) == 0) {
      s_wbl[w] = wl;
      s_wbh[w] = wh;
    }
  }
  __syncthreads();
  if (t == 0) {
    int blo = kHistBins, bhi = kHistBins;
#pragma unroll
    for (int u = 0; u < kTopWaves; ++u) {
      blo = min(blo, s_wbl[u]);
      bhi = min(bhi, s_wbh[u]);
    }
    TopBand tb;
    tb.z = Z;
    tb.m = M;
    // the bound never reaching top_p would mean the counts missed mass:
    // the fallback decides such a row
    tb.state = blo == kHistBins || s_sat ? kTopFallback : kTopCounts;
    tb.blo = blo;
    tb.bhi = bhi == kHistBins ? kHistBins - 1 : bhi;
    a.topband[row] = tb;
  }
}

// ---------------------------------------------------------------------------
// gather: per row, the exact mass above the band and the band's keys
// ---------------------------------------------------------------------------
constexpr int kGWin = kTopThreads / 16;             // splits per window (16 lanes a split's scalars)
constexpr int kGWinEnt = kGWin * kChunksPerSplit;   // chunk entries per window
constexpr int kGRounds = kGWinEnt / (8 * kTopThreads);  // 16-byte loads of entries per lane
// chunk lines per lane group and pass: 8 for fp32; 2 for bf16 (eight slots
// of eight bf16 elements took 214 registers, one workgroup per CU; two take
// 95, and the bf16 top-p call ran 577 -> 564 us at B256 K4 V152064)
template <int DT>
constexpr int gather_slots() { return DT == kBF16 ? 2 : 8; }
constexpr int kGQueue = 192;     // vectors queued per wave before they are classified
constexpr int kGWaveKeys = 256;  // band keys a wave holds per pass

// rank of the calling lane among the lanes set in `bal` below it
__device__ __forceinline__ unsigned lane_rank(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// Exclusive prefix of v over the workgroup; *total gets the sum.  Whole
// workgroup; wtot is free again on return.
__device__ __forceinline__ int block_excl_scan(int v, int *wtot, int *total) {
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int incl = wave_incl_scan(v);
  if (l == 63) wtot[w] = incl;
  __syncthreads();
  int before = incl - v, sum = 0;
#pragma unroll
  for (int u = 0; u < kTopWaves; ++u) {
    if (u < w) before += wtot[u];
    sum += wtot[u];
  }
  __syncthreads();
  *total = sum;
  return before;
}

// One workgroup per row, over windows of kGWin splits.  The window's chunk
// records classify the 128-byte lines: a chunk whose maximum c has c kk <
// F - bhi holds no element at or above the band (x <= c and kk > 0 give x
// kk <= c kk, rounding keeps the order); a chunk whose second largest
// element lies below the band holds exactly one, its maximum, which the
// record gives exactly; only the remaining chunks are read: their indices
// are packed into LDS, and passes of kGPerPass lines, each line read by a
// group of eight lanes, visit only those.  Every split's scalar head and
// tail elements are visited too.  Each wave appends its band keys in a
// fixed order, and the waves' lists go to the row's list in wave order,
// with no atomics.
template <int DT>
__global__ __launch_bounds__(kTopThreads, 6) void k_topp_gather(SampleArgs a) {
  const int row = blockIdx.x, S = a.S, t = threadIdx.x;
  const TopRow tr = top_row<DT>(a, row);
  if (tr.q.invalid || tr.q.greedy || !(tr.q.top_p < 1.0)) return;
  // a row the counts did not cover is decided by the cut launch
  const TopBand tb = a.topband[row];
  if (tb.state != kTopCounts) return;
  const Scale k = tr.q.k;
  const float kk = (k.hi + k.lo) * kHistPerLog2;
  const float M = tb.m, F = floorf(M * kk);
  constexpr int EPV = 16 / elem_bytes(DT);
  static_assert(2 * (EPV - 1) <= 16, "a split's scalars fit its 16 lanes");
  // With y = x kk (the product grid_bin floors): bin < blo iff y >= F - blo
  // + 1, bin <= bhi iff y >= F - bhi (integers, exact in fp32 below 2^24),
  // so an element below the band costs one product and one compare.
  const float ya = F - (float)tb.blo + 1.f, yb = F - (float)tb.bhi;

  __shared__ uint16_t list[kGWinEnt];
  __shared__ int wtot[kTopWaves];
  __shared__ double wsum[kTopWaves];
  __shared__ u32x4 gq[kTopWaves][kGQueue];         // per wave: queued vectors
  __shared__ uint32_t gkeys[kTopWaves][kGWaveKeys];  // per wave: the pass's band keys
  __shared__ int gkn[kTopWaves];
  const int w = t >> 6, lane = t & 63;
  uint32_t *keys = a.band_keys + (size_t)row * kBandKeys;
  const uint32_t *cm = a.part_c + (size_t)row * S * kChunksPerSplit;
  const uint16_t *cm2 = a.part_c2 + (size_t)row * S * kChunksPerSplit;
  double above = 0.0;
  int kbase = 0;  // keys of the passes before (uniform)
  int kn = 0;     // the wave's band keys in this pass (uniform in the wave)
  bool lost = false;
  // split bodies: splits start 32 KB apart, so every full split has the
  // first one's head and vector count; the last has its own count
  const Span sp0 = split_span(tr.rp, a.V, 0, DT), spl = split_span(tr.rp, a.V, S - 1, DT);
  const u32x4 *body0 = span_body(sp0, DT);
  constexpr int kSplitVecs = kThreads * kVecPerThread;

  for (int s0 = 0; s0 < S; s0 += kGWin) {
    const int sw = min(kGWin, S - s0), nent = sw * kChunksPerSplit;
    // the window's chunk maxima and second-element bounds, eight entries a
    // lane and round ...
    u32x4 c1w[kGRounds][2], c2w[kGRounds];
#pragma unroll
    for (int r = 0; r < kGRounds; ++r) {
      const int e = (r * kTopThreads + t) * 8;
      if (e < nent) {
        const size_t at = (size_t)s0 * kChunksPerSplit + e;
        c1w[r][0] = *reinterpret_cast<const u32x4 *>(cm + at);
        c1w[r][1] = *reinterpret_cast<const u32x4 *>(cm + at + 4);
        c2w[r] = *reinterpret_cast<const u32x4 *>(cm2 + at);
      } else {
        c1w[r][0] = c1w[r][1] = neg_inf_vec<kF32>();
        c2w[r] = neg_inf_vec<kBF16>();
      }
    }
    // ... and each split's scalars (lanes 16 j .. 16 j + 15 for split s0 + j)
    float xs = -INFINITY;
    {
      const int j = t >> 4, q = t & 15;
      if (j < sw) {
        const Span sp = split_span(tr.rp, a.V, s0 + j, DT);
        const int se = span_scalar_elem(sp, q, DT);
        if (se >= 0) xs = load_elem(sp.base, se, DT);
      }
    }
    // A line holds an element at or above the band iff its maximum c1 does.
    // If its second largest element lies below the band, c1 is the only
    // one, and its value (recorded exactly) is all the band needs: its mass
    // if above the band, else its key (appended to the wave's key list in
    // lane order), with no read of the line.  Only lines with two or more
    // such elements (about one in fifty) go into the list.
    uint32_t bits[kGRounds];
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < kGRounds; ++r) {
      bits[r] = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float c1 = __uint_as_float(c1w[r][j >> 2][j & 3]);
        const float c2 = __uint_as_float(((c2w[r][j >> 1] >> (16 * (j & 1))) & 0xFFFFu) << 16);
        const float y1 = c1 * kk;
        const bool cand = y1 >= yb;
        const bool many = cand && !(c2 * kk < yb);
        bits[r] |= many ? 1u << j : 0u;
        const bool one = cand && !many;
        if (one && y1 >= ya) above += (double)tempered(c1, M, k);
        const bool inb = one && y1 < ya;
        const uint64_t bal = __ballot(inb);
        const int kp = kn + (int)lane_rank(bal);
        if (inb && kp < kGWaveKeys) gkeys[w][kp] = key_of_f32(c1);
        kn += __popcll(bal);
      }
      cnt += __builtin_popcount(bits[r]);
    }
    int n;
    int pos = block_excl_scan(cnt, wtot, &n);
#pragma unroll
    for (int r = 0; r < kGRounds; ++r) {
      const int e0 = (r * kTopThreads + t) * 8;
      for (uint32_t b = bits[r]; b; b &= b - 1u) list[pos++] = (uint16_t)(e0 + __builtin_ctz(b));
    }
    __syncthreads();

    // passes over the listed lines: lane group t / 8 takes items t / 8 +
    // 64 r, lane t one 16-byte vector of each (entry g * 8 + u of a split
    // is its vectors 8 g .. 8 g + 7 of slot u: v = 8 g + lane + u kThreads)
    constexpr int kGSlots = gather_slots<DT>();
    constexpr int kGPerPass = kTopThreads / kChunkLanes * kGSlots;
    for (int p0 = 0; p0 == 0 || p0 < n; p0 += kGPerPass) {
      // every list read first, then every load
      int ent[kGSlots];
#pragma unroll
      for (int r = 0; r < kGSlots; ++r) {
        const int i = p0 + r * (kTopThreads / kChunkLanes) + t / kChunkLanes;
        ent[r] = i < n ? (int)list[i] : -1;
      }
      u32x4 buf[kGSlots];
#pragma unroll
      for (int r = 0; r < kGSlots; ++r) {
        buf[r] = neg_inf_vec<DT>();
        if (ent[r] >= 0) {
          const int sp = s0 + ent[r] / kChunksPerSplit, e = ent[r] % kChunksPerSplit;
          const int v = (e / kVecPerThread) * kChunkLanes + (t % kChunkLanes) + (e % kVecPerThread) * kThreads;
          if (v < (sp == S - 1 ? spl.nvec : sp0.nvec))
            buf[r] = load_stream(body0 + (size_t)sp * kSplitVecs + v);
        }
      }
      // A listed line holds about one element at or above the band in
      // thirty-two, scattered over the lanes, so classifying every element
      // in place would run the mass and key code for nearly every element
      // with a lane or two active.  Instead each wave first queues, in LDS,
      // the vectors whose maximum reaches the band (one product and one
      // compare per vector), then classifies the queue with every lane busy.
      int qn = 0;  // queued vectors (uniform in the wave)
      auto drain = [&]() {
        for (int i0 = 0; i0 < qn; i0 += 64) {
          const int i = i0 + lane;
          const u32x4 v = i < qn ? gq[w][i] : neg_inf_vec<DT>();
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const float x = vec_elem(v, e, DT);
            const float y = x * kk;
            if (y >= ya) above += (double)tempered(x, M, k);
            const bool inb = y >= yb && y < ya;
            const uint64_t bal = __ballot(inb);
            const int pos = kn + (int)lane_rank(bal);
            if (inb && pos < kGWaveKeys) gkeys[w][pos] = key_of_f32(x);
            kn += __popcll(bal);
          }
        }
        qn = 0;
      };
      auto push = [&](const u32x4 &v, float vmax) {
        if (qn > kGQueue - 64) drain();
        const bool hit = vmax * kk >= yb;
        const uint64_t bal = __ballot(hit);
        if (hit) gq[w][qn + (int)lane_rank(bal)] = v;
        qn += __popcll(bal);
      };
#pragma unroll
      for (int r = 0; r < kGSlots; ++r) {
        float vmax = vec_elem(buf[r], 0, DT);
#pragma unroll
        for (int e = 1; e < EPV; ++e) vmax = fmaxf(vmax, vec_elem(buf[r], e, DT));
        push(buf[r], vmax);
      }
      if (p0 == 0) {  // the splits' scalar elements, as vectors of one element
        u32x4 v = neg_inf_vec<DT>();
        v[0] = DT == kBF16 ? (v[0] & 0xFFFF0000u) | (__float_as_uint(xs) >> 16) : __float_as_uint(xs);
        push(v, xs);
      }
      drain();
      // the wave's band keys of this pass go to the row's list after the
      // keys of the waves before it (workgroup order: the same on every run)
      if (lane == 0) gkn[w] = kn;
      __syncthreads();
      int off = kbase, tot = 0;
#pragma unroll
      for (int u = 0; u < kTopWaves; ++u) {
        const int c = gkn[u];
        off += u < w ? c : 0;
        tot += c;
        lost |= c > kGWaveKeys;
      }
      for (int i = lane; i < min(kn, kGWaveKeys); i += 64)
        if (off + i < kBandKeys) keys[off + i] = gkeys[w][i];
      kbase += tot;
      kn = 0;
      __syncthreads();  // the queue and key lists are refilled by the next pass
    }
    __syncthreads();  // the list and split table are rewritten by the next window
  }
  const double wa = wave_sum(above);
  if ((t & 63) == 0) wsum[t >> 6] = wa;
  __syncthreads();
  if (t == 0) {
    double sum = 0.0;
#pragma unroll
    for (int u = 0; u < kTopWaves; ++u) sum += wsum[u];
    a.band_above[row] = sum;
    // a wave that found more band keys in one pass than its LDS list holds
    // dropped some: the cut then reads the row instead of the list
    a.band_n[row] = lost ? (unsigned)max(kbase, kBandKeys + 1) : (unsigned)kbase;
  }
}

// ---------------------------------------------------------------------------
// cut: per row, the radix rounds (and the fallback for uncovered rows)
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kTopThreads, 8) void k_topp_cut(SampleArgs a) {
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int V = a.V;
  const TopRow tr = top_row<DT>(a, row);
  if (tr.q.invalid || tr.q.greedy) return;
  const TopBand tb = a.topband[row];
  if (tb.state == kTopDone) return;
  const char *rp = tr.rp;
  const Scale k = tr.q.k;
  const double top_p = tr.q.top_p;
  const float M = tb.m;
  const double Z = tb.z;
  const double goal = top_p * Z;
  const float kk = (k.hi + k.lo) * kHistPerLog2;
  const float kr = (k.hi + k.lo) * kBinsPerLog2;
  const bool fast = tb.state == kTopCounts;
  const float F = floorf(M * kk);
  const int blo = tb.blo, bhi = tb.bhi;

  __shared__ double hist[kTopWaves][kBins];
  __shared__ double mass[kBins];
  __shared__ unsigned cnt[kBins], kmin[kBins], kmax[kBins];
  __shared__ double s_above;
  __shared__ int s_bin, s_done;
  __shared__ unsigned s_prefix;
  __shared__ float s_tau;
  __shared__ double s_kept;
  __shared__ uint32_t cand[kCand];
  __shared__ unsigned s_ncand;
  int sel = -1;

  if (fast) {
    // the band's keys and the exact mass above them, from the gather tiles
    const unsigned n = a.band_n[row];
    if (t == 0) {
      const double sum = a.band_above[row];
      s_above = sum;
      s_kept = sum;
      s_done = 0;
      s_prefix = 0;
      s_tau = -INFINITY;
      s_ncand = n;
    }
    if (n <= (unsigned)kCand) {
      const uint32_t *keys = a.band_keys + (size_t)row * kBandKeys;
      for (unsigned i = t; i < n; i += kTopThreads) cand[i] = keys[i];
    }
    __syncthreads();
  } else {
    if (t == 0) s_ncand = 0;
    for (int i = t; i < kTopWaves * kBins; i += kTopThreads) (&hist[0][0])[i] = 0.0;
    __syncthreads();
    // fallback 1. mass by distance bin; the last bin (everything beyond
    //    it, where most of a long tail sits) is summed in registers instead
    //    of LDS atomics
    {
      double far = 0.0;
      for_row<DT>(rp, V, [&](int, float x) {
        const int bin = dist_bin(x, M, kr);
        const double tm = (double)tempered(x, M, k);
        if (bin < kBins - 1)
          atomicAdd(&hist[w][bin], tm);
        else
          far += tm;
      });
      far = wave_sum(far);
      __syncthreads();
      if ((t & 63) == 0) hist[w][kBins - 1] += far;
    }
    __syncthreads();
    if (t < kBins) {
      double sum = 0.0;
      for (int u = 0; u < kTopWaves; ++u) sum += hist[u][t];
      mass[t] = sum;
    }
    __syncthreads();
    if (t == 0) {
      double cum = 0.0;
      int sl = -1;
      for (int bb = 0; bb < kBins; ++bb) {
        if (cum + mass[bb] >= goal) {
          sl = bb;
          break;
        }
        cum += mass[bb];
      }
      s_bin = sl;
      s_above = cum;
      s_prefix = 0;
      s_done = sl < 0;  // the cumulative mass never reached top_p: keep everything
      s_tau = -INFINITY;
      s_kept = sl < 0 ? Z : cum;
    }
    __syncthreads();
    // fallback 2. the selected bin's elements, gathered into LDS as value
    //    keys: each thread counts its elements of the bin, then writes them
    //    at offsets from a workgroup scan (two more passes over the row; the
    //    keys land in the same order on every run)
    sel = s_bin;
    if (!s_done) {
      __shared__ int wtot[kTopWaves];
      int mine = 0, total = 0;
      for_row<DT>(rp, V, [&](int, float x) { mine += dist_bin(x, M, kr) == sel; });
      int slot = block_excl_scan(mine, wtot, &total);
      for_row<DT>(rp, V, [&](int, float x) {
        if (dist_bin(x, M, kr) != sel) return;
        if (slot < kCand) cand[slot] = key_of_f32(x);
        ++slot;
      });
      if (t == 0) s_ncand = (unsigned)total;
      __syncthreads();
    }
  }
  const unsigned ncand = s_ncand;
  const bool in_lds = ncand <= (unsigned)kCand;

  // keys held in LDS: the rounds start at the first byte where the smallest
  // and largest key differ (a round above it would find one non-empty bin
  // and add no mass above it)
  int shift0 = 24;
  if (in_lds && ncand > 0) {
    __shared__ uint32_t s_klo, s_khi;
    if (t == 0) {
      s_klo = 0xFFFFFFFFu;
      s_khi = 0u;
    }
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (unsigned i = t; i < ncand; i += kTopThreads) {
      lo = min(lo, cand[i]);
      hi = max(hi, cand[i]);
    }
    hi = (uint32_t)wave_max_u64(hi);
    lo = ~(uint32_t)wave_max_u64((uint64_t)~lo);
    __syncthreads();
    if (lane_id() == 0) {
      atomicMin(&s_klo, lo);
      atomicMax(&s_khi, hi);
    }
    __syncthreads();
    const uint32_t d = s_klo ^ s_khi;
    shift0 = d ? ((31 - __builtin_clz(d)) >> 3) << 3 : 0;
    if (t == 0 && shift0 < 24) s_prefix = s_klo >> (shift0 + 8);
    __syncthreads();
  }

  // exact cut among the gathered keys (the band, or the selected bin):
  // radix rounds over value keys, accumulating mass from the top; if they
  // did not fit in LDS, each round reads the row again.  Each wave adds its
  // keys' masses into its own row of bins (a wave's adds come in program
  // order), and the rows are summed in wave order, so the kept mass is the
  // same bit for bit on every run; the counts and key bounds are integers.
  __shared__ double exc[kBins], rtot[kBins / 64];
  __shared__ int s_wfirst[kBins / 64], s_wlast[kBins / 64];
  for (int shift = shift0; shift >= 0 && !s_done; shift -= 8) {
    for (int i = t; i < kTopWaves * kBins; i += kTopThreads) (&hist[0][0])[i] = 0.0;
    if (t < kBins) {
      cnt[t] = 0;
      kmin[t] = 0xFFFFFFFFu;
      kmax[t] = 0u;
    }
    __syncthreads();
    const unsigned prefix = s_prefix;
    auto visit = [&](uint32_t key) {
      if (shift < 24 && (key >> (shift + 8)) != prefix) return;
      const int sb = (key >> shift) & 0xFF;
      atomicAdd(&hist[w][sb], (double)tempered(f32_of_key(key), M, k));
      atomicAdd(&cnt[sb], 1u);
      atomicMin(&kmin[sb], key);
      atomicMax(&kmax[sb], key);
    };
    if (in_lds) {
      for (unsigned i = t; i < ncand; i += kTopThreads) visit(cand[i]);
    } else {
      for_row<DT>(rp, V, [&](int, float x) {
        if (fast) {
          const int bin = grid_bin(x, F, kk);
          if (bin >= blo && bin <= bhi) visit(key_of_f32(x));
        } else if (dist_bin(x, M, kr) == sel) {
          visit(key_of_f32(x));
        }
      });
    }
    __syncthreads();
    if (t < kBins) {
      double sum = 0.0;
#pragma unroll
      for (int u = 0; u < kTopWaves; ++u) sum += hist[u][t];
      mass[t] = sum;
    }
    __syncthreads();
    // from the top bin down (lane t: bin 255 - t), the mass of the
    // non-empty bins above each one; the pick is the first non-empty bin
    // where the mass so far reaches the goal (if rounding leaves none, the
    // last non-empty bin closes the nucleus)
    double v = 0.0;
    bool nz = false;
    if (t < kBins) {
      nz = cnt[kBins - 1 - t] != 0u;
      v = nz ? mass[kBins - 1 - t] : 0.0;
    }
    const double incl = wave_incl_scan(v);
    if (t < kBins && (t & 63) == 63) rtot[t >> 6] = incl;
    __syncthreads();
    bool reach = false;
    if (t < kBins) {
      double ex = incl - v;
#pragma unroll
      for (int u = 0; u < kBins / 64; ++u)
        if (u < (t >> 6)) ex += rtot[u];
      exc[t] = ex;
      reach = nz && s_above + ex + v >= goal;
    }
    // the first lane that reaches the goal and the last non-empty one, per
    // wave (lanes ascend with t)
    const uint64_t hr = __ballot(reach), hn = __ballot(nz);
    if (t < kBins && (t & 63) == 0) {
      s_wfirst[w] = hr ? (t & ~63) + (int)__builtin_ctzll(hr) : kBins;
      s_wlast[w] = hn ? (t & ~63) + 63 - (int)__builtin_clzll(hn) : -1;
    }
    __syncthreads();
    if (t == 0) {
      int first = kBins, lastnz = -1;
#pragma unroll
      for (int u = 0; u < kBins / 64; ++u) {
        first = min(first, s_wfirst[u]);
        lastnz = max(lastnz, s_wlast[u]);
      }
      const int pt = first < kBins ? first : lastnz;
      if (pt < 0) {  // nothing gathered: cannot happen; keep everything
        s_done = 1;
        s_tau = -INFINITY;
        s_kept = Z;
        s_above = 0.0;
      } else {
        const int pick = kBins - 1 - pt;
        const double above = s_above + exc[pt];
        s_above = above;
        s_prefix = (prefix << 8) | (unsigned)pick;
        if (kmin[pick] == kmax[pick] || shift == 0) {
          s_done = 1;
          s_tau = f32_of_key(kmin[pick]);
          s_kept = above + mass[pick];
        }
      }
    }
    __syncthreads();
  }
  if (t == 0) {
    RowStat rs;
    rs.m = M;
    rs.z = Z;
    rs.tau = s_tau;
    rs.zk = s_kept;
    a.rowstat[row] = rs;
  }
}

hipError_t launch_topp_select(const SampleArgs &a, int dtype, hipStream_t stream) {
  const int rows = a.B * (2 * a.K + 1);
  if (dtype == kBF16) {
    hipLaunchKernelGGL(k_topp_band<kBF16>, dim3(rows), dim3(kTopThreads), 0, stream, a);
    hipLaunchKernelGGL(k_topp_gather<kBF16>, dim3(rows), dim3(kTopThreads), 0, stream, a);
    hipLaunchKernelGGL(k_topp_cut<kBF16>, dim3(rows), dim3(kTopThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(k_topp_band<kF32>, dim3(rows), dim3(kTopThreads), 0, stream, a);
    hipLaunchKernelGGL(k_topp_gather<kF32>, dim3(rows), dim3(kTopThreads), 0, stream, a);
    hipLaunchKernelGGL(k_topp_cut<kF32>, dim3(rows), dim3(kTopThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace sv
