// Top-p (nucleus) threshold per logit row, exact, without a sort.
//
// After temperature, keep the largest logits, whole tie groups, until their
// mass first reaches top_p of the row, and renormalise (ariser.io review,
// section "같은 분포를 지키는 작은 장치": temperature / top-p must be applied
// to both p and q before the test; the nucleus rule itself is the plainest
// reading, the pages name it only).  With the row maximum M and the
// normaliser Z known from the streaming pass, one workgroup per row:
//   1. builds an LDS histogram of tempered mass over bins of the distance
//      (M - l) * log2(e)/T, 1/8 log2 unit wide (per-wave copies, fp64);
//      scanning from the nearest bin finds the bin where the cumulative mass
//      reaches top_p * Z; bins are value intervals, so tie groups never split;
//   2. resolves the exact cut inside that bin by radix rounds of 8 bits over
//      order-preserving value keys, again accumulating mass from the top,
//      until one distinct value remains: that value is tau, the mass at or
//      above it is the kept mass.
#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {

constexpr int kTopThreads = 512;
constexpr int kTopWaves = kTopThreads / 64;
constexpr int kBins = 256;
constexpr float kBinsPerLog2 = 8.f;
constexpr int kCand = 4096;  // keys of the selected bin held in LDS

namespace {

__device__ __forceinline__ int dist_bin(float x, float M, float kr) {
  const float d = (M - x) * kr;   // >= 0; +inf for x = -inf
  return d < (float)(kBins - 1) ? (int)d : kBins - 1;
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

}  // namespace

template <int DT>
__global__ __launch_bounds__(kTopThreads) void k_topp_select(SampleArgs a) {
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int V = a.V, S = a.S;
  const int rows_t = a.B * (a.K + 1);
  const size_t row_bytes = (size_t)V * elem_bytes(DT);
  const char *rp = row < rows_t ? a.target + (size_t)row * row_bytes
                                : a.draft + (size_t)(row - rows_t) * row_bytes;
  const int b = row < rows_t ? row / (a.K + 1) : (row - rows_t) / a.K;
  const ReqParams q = request_params(a.temps, a.topps, a.k64, a.k, a.top_p, b);
  if (q.invalid || q.greedy) return;  // no softmax statistics for this request
  const Scale k = q.k;
  const double k64 = q.k64, top_p = q.top_p;
  const u64 *part_m = a.part_m, *part_z = a.part_z;
  RowStat *rowstat = a.rowstat;

  __shared__ double hist[kTopWaves][kBins];
  __shared__ double mass[kBins];
  __shared__ unsigned cnt[kBins], kmin[kBins], kmax[kBins];
  __shared__ float sM;
  __shared__ double sZ, s_above;
  __shared__ int s_bin, s_done;
  __shared__ unsigned s_prefix;
  __shared__ float s_tau;
  __shared__ double s_kept;
  __shared__ uint32_t cand[kCand];
  __shared__ unsigned s_ncand;

  if (t == 0) {  // the streaming kernel has completed: every partial is in place
    const u64 *pm = part_m + (size_t)row * S;
    const u64 *pz = part_z + (size_t)row * S * 2;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, payload_f32(pm[s]));
    double Z = 0.0;
    for (int s = 0; s < S; ++s) {
      const float m = payload_f32(pm[s]);
      const double z = (double)payload_f32(pz[2 * s]) + (double)payload_f32(pz[2 * s + 1]);
      if (m > -INFINITY) Z += z * exp2(((double)m - (double)M) * k64);
    }
    sM = M;
    sZ = Z;
  }
  for (int i = t; i < kTopWaves * kBins; i += kTopThreads) (&hist[0][0])[i] = 0.0;
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
      rowstat[row] = rs;
    }
    return;
  }
  const double goal = top_p * Z;
  const float kr = (k.hi + k.lo) * kBinsPerLog2;

  // 1. mass by distance bin; the last bin (everything beyond it, where most
  //    of a long tail sits) is summed in registers instead of LDS atomics
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
    double s = 0.0;
    for (int u = 0; u < kTopWaves; ++u) s += hist[u][t];
    mass[t] = s;
  }
  __syncthreads();
  if (t == 0) {
    double cum = 0.0;
    int sel = -1;
    for (int b = 0; b < kBins; ++b) {
      if (cum + mass[b] >= goal) {
        sel = b;
        break;
      }
      cum += mass[b];
    }
    s_bin = sel;
    s_above = cum;
    s_prefix = 0;
    s_done = sel < 0;  // the cumulative mass never reached top_p: keep everything
    s_tau = -INFINITY;
    s_kept = cum;
  }
  __syncthreads();

  // 2. the selected bin's elements, gathered into LDS as value keys (one
  //    more pass over the row); if they do not fit, the rounds below read
  //    the row again each time
  const int sel = s_bin;
  if (!s_done) {
    if (t == 0) s_ncand = 0;
    __syncthreads();
    for_row<DT>(rp, V, [&](int, float x) {
      if (dist_bin(x, M, kr) != sel) return;
      const unsigned slot = atomicAdd(&s_ncand, 1u);
      if (slot < (unsigned)kCand) cand[slot] = key_of_f32(x);
    });
    __syncthreads();
  }
  const unsigned ncand = s_ncand;
  const bool in_lds = ncand <= (unsigned)kCand;

  // 3. exact cut inside the selected bin: radix rounds over value keys,
  //    accumulating mass from the top
  for (int shift = 24; shift >= 0 && !s_done; shift -= 8) {
    if (t < kBins) {
      mass[t] = 0.0;
      cnt[t] = 0;
      kmin[t] = 0xFFFFFFFFu;
      kmax[t] = 0u;
    }
    __syncthreads();
    const unsigned prefix = s_prefix;
    auto visit = [&](uint32_t key) {
      if (shift < 24 && (key >> (shift + 8)) != prefix) return;
      const int sb = (key >> shift) & 0xFF;
      atomicAdd(&mass[sb], (double)tempered(f32_of_key(key), M, k));
      atomicAdd(&cnt[sb], 1u);
      atomicMin(&kmin[sb], key);
      atomicMax(&kmax[sb], key);
    };
    if (in_lds) {
      for (unsigned i = t; i < ncand; i += kTopThreads) visit(cand[i]);
    } else {
      for_row<DT>(rp, V, [&](int, float x) {
        if (dist_bin(x, M, kr) == sel) visit(key_of_f32(x));
      });
    }
    __syncthreads();
    if (t == 0) {
      double above = s_above;
      int pick = -1;
      for (int sb = kBins - 1; sb >= 0; --sb) {
        if (!cnt[sb]) continue;
        if (above + mass[sb] >= goal) {
          pick = sb;
          break;
        }
        above += mass[sb];
      }
      if (pick < 0) {  // rounding: the bin's last group closes the nucleus
        above = s_above;
        for (int sb = kBins - 1; sb >= 0; --sb) {
          if (!cnt[sb]) continue;
          pick = sb;
          above += mass[sb];
        }
        if (pick >= 0) above -= mass[pick];
      }
      if (pick < 0) {  // no element in the bin: cannot happen; keep everything
        s_done = 1;
        s_tau = -INFINITY;
        s_kept = Z;
        s_above = 0.0;
      } else {
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
    if (sel < 0) {
      rs.tau = -INFINITY;
      rs.zk = Z;
    } else {
      rs.tau = s_tau;
      rs.zk = s_kept;
    }
    rowstat[row] = rs;
  }
}

hipError_t launch_topp_select(const SampleArgs &a, int dtype, hipStream_t stream) {
  dim3 grid(a.B * (2 * a.K + 1)), block(kTopThreads);
  if (dtype == kBF16)
    hipLaunchKernelGGL(k_topp_select<kBF16>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(k_topp_select<kF32>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace sv
