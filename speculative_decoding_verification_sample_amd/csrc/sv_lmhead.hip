// The target's LM head fused in front of greedy verification: logits =
// hidden states x vocabulary matrix^T on the matrix cores, reduced to each
// row's top choice without ever writing the logits (lotook.com explainer,
// the four steps: one target pass yields the K+1 distributions, and the
// greedy rule of its FAQ accepts a draft only if it is the top choice).
//
// k_lmhead_argmax: one workgroup (4 waves) per 384-row x 128-column tile of
// the logits (all the rows of a verify call fit one tile, so the vocabulary
// matrix is read once), d reduced in stages of 32 through double-buffered
// LDS with v_mfma_f32_32x32x16_bf16 (fp32 accumulation of exact bf16
// products).  Each wave owns 192 rows x 64 columns (6 x 2 blocks of 32 x 32).
// LDS holds a stage as [k chunk of 8][row or column] 16-byte entries, so
// that the 32 lanes reading one operand fragment touch 512 contiguous bytes.
// The epilogue finds each row's best (value, lowest column) through an LDS
// transpose and keeps one 64-bit key per (row, vocabulary tile).
// k_lmhead_decide: one workgroup per request combines its rows' partials and
// applies the greedy rule.
#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLmRows = 384;   // rows per tile (12 blocks of 32)
constexpr int kLmCols = 128;   // vocabulary columns per tile (4 blocks of 32)
constexpr int kLmK = 32;       // d per LDS stage
constexpr int kLmChunks = kLmK / 8;
constexpr int kLmWaveRows = kLmRows / 2;  // each wave: 192 rows x 64 columns
constexpr int kLmRB = kLmWaveRows / 32;   // 6 row blocks per wave
constexpr int kLmA = kLmRows * kLmChunks / 256;  // staged 16-byte loads per thread: 6
constexpr int kLmB = kLmCols * kLmChunks / 256;  // 2

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

struct StageA {
  u32x4 v[kLmA];
};
struct StageB {
  u32x4 v[kLmB];
};

}  // namespace

__global__ __launch_bounds__(256) void k_lmhead_argmax(const u32x4 *__restrict__ hidden,
                                                       const u32x4 *__restrict__ weight,
                                                       int M, int d, int V, int RT, int VT,
                                                       uint64_t *__restrict__ part) {
  // block -> (vocabulary tile vt, row tile rt): the RT row tiles of one
  // vocabulary tile share blockIdx mod 8 (one XCD) and run back to back
  const int blk = blockIdx.x;
  const int grp = blk / (8 * RT), rem = blk - grp * 8 * RT;
  const int rt = rem >> 3, vt = grp * 8 + (rem & 7);
  if (vt >= VT) return;
  const int r0 = rt * kLmRows, v0 = vt * kLmCols;
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int wr = wv >> 1, wc = wv & 1;  // wave's 192-row and 64-column part
  const int dv = d >> 3;                // 16-byte chunks per row

  // one buffer: A [chunk][row], B [chunk][column], 16-byte entries (the 32
  // lanes reading a fragment touch 512 contiguous bytes); the chunk planes
  // are two entries longer than a row of entries, so that the 8 lanes of a
  // store group (2 rows x 4 chunks) spread over 32 banks
  constexpr int kPA = kLmRows + 2, kPB = kLmCols + 2;  // plane strides (entries)
  __shared__ u32x4 sA[2][kLmChunks * kPA];
  __shared__ u32x4 sB[2][kLmChunks * kPB];
  __shared__ uint64_t sKey[2][kLmRows];

  // staging: entry e = t + 256 j -> (row or column e / 4, chunk e % 4): 4
  // lanes read a row's 64 bytes of the stage.  Rows at or past M and
  // columns at or past V load row M-1 / column V-1 (unconditional loads keep
  // the wait counts exact); their products only reach rows that are never
  // written and columns the epilogue drops.
  const u32x4 *hp[kLmA], *wp[kLmB];
#pragma unroll
  for (int j = 0; j < kLmA; ++j) {
    const int e = t + 256 * j;
    hp[j] = hidden + (size_t)min(r0 + (e >> 2), M - 1) * dv + (e & 3);
  }
#pragma unroll
  for (int j = 0; j < kLmB; ++j) {
    const int e = t + 256 * j;
    wp[j] = weight + (size_t)min(v0 + (e >> 2), V - 1) * dv + (e & 3);
  }
  auto load_a = [&](int s, StageA &R) {
#pragma unroll
    for (int j = 0; j < kLmA; ++j) R.v[j] = hp[j][s * kLmChunks];
  };
  auto load_b = [&](int s, StageB &R) {
#pragma unroll
    for (int j = 0; j < kLmB; ++j) R.v[j] = __builtin_nontemporal_load(wp[j] + s * kLmChunks);
  };
  auto store = [&](int buf, const StageA &A, const StageB &B) {
#pragma unroll
    for (int j = 0; j < kLmA; ++j) {
      const int e = t + 256 * j;
      sA[buf][(e & 3) * kPA + (e >> 2)] = A.v[j];
    }
#pragma unroll
    for (int j = 0; j < kLmB; ++j) {
      const int e = t + 256 * j;
      sB[buf][(e & 3) * kPB + (e >> 2)] = B.v[j];
    }
  };

  f32x16 acc[kLmRB][2];
#pragma unroll
  for (int i = 0; i < kLmRB; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][c][v] = 0.f;

  // all operand fragments of the stage's two k-steps are read first, then
  // the 24 products issue back to back
  auto compute = [&](int buf) {
    bf16x8 fa[2][kLmRB], fb[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ks * 2 + (l >> 5);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        fb[ks][c] = as_bf16x8(sB[buf][ch * kPB + wc * 64 + c * 32 + (l & 31)]);
#pragma unroll
      for (int i = 0; i < kLmRB; ++i)
        fa[ks][i] = as_bf16x8(sA[buf][ch * kPA + wr * kLmWaveRows + i * 32 + (l & 31)]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < kLmRB; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][i], fb[ks][c], acc[i][c], 0, 0, 0);
    // scheduling hint: the 16 fragment reads first, then the 24 products
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 24, 0);
  };

  // The vocabulary matrix streams from HBM with four stages in flight; the
  // hidden states (a few MB, read by every tile) come from L2 two stages
  // ahead.  A step: the sets that held stage s (stored by the step before)
  // take stage s + 4 / s + 2 (the last stage again near the end), stage s is
  // multiplied, stage s + 1 is stored (past the end, a copy of the last
  // stage lands in a buffer nothing reads).
  const int S = d / kLmK;
  StageA H0, H1;
  StageB W0, W1, W2, W3;
  auto step = [&](int s, StageB &wcur, StageB &wnext, StageA &hcur, StageA &hnext) {
    load_b(min(s + 4, S - 1), wcur);
    load_a(min(s + 2, S - 1), hcur);
    compute(s & 1);
    store((s + 1) & 1, hnext, wnext);
    __syncthreads();
  };
  load_b(0, W0);
  load_a(0, H0);
  load_b(min(1, S - 1), W1);
  load_a(min(1, S - 1), H1);
  load_b(min(2, S - 1), W2);
  load_b(min(3, S - 1), W3);
  store(0, H0, W0);
  __syncthreads();
  int s = 0;
  for (; s + 4 <= S; s += 4) {
    step(s, W0, W1, H0, H1);
    step(s + 1, W1, W2, H1, H0);
    step(s + 2, W2, W3, H0, H1);
    step(s + 3, W3, W0, H1, H0);
  }
  if (s < S) step(s, W0, W1, H0, H1);
  if (s + 1 < S) step(s + 1, W1, W2, H1, H0);
  if (s + 2 < S) step(s + 2, W2, W3, H0, H1);

  // epilogue: each row's best (value, lowest column).  Per row block the
  // wave writes its 32 x 64 logits to LDS (the operand buffers are free
  // now), then lane l scans columns 32 (l / 32) .. + 32 of row l % 32, and
  // the two halves combine through one lane exchange.
  float *sT = reinterpret_cast<float *>(&sA[0][0]) + wv * (32 * 65);
#pragma unroll
  for (int i = 0; i < kLmRB; ++i) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        sT[row * 65 + c * 32 + (l & 31)] = acc[i][c][v];
      }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const int row = l & 31, half = l >> 5;
    const int cbase = v0 + wc * 64 + half * 32;
    float bv = -INFINITY;
    int bc = 0x7FFFFFFF;
    for (int j = 0; j < 32; ++j) {
      const float x = cbase + j < V ? sT[row * 65 + half * 32 + j] : -INFINITY;
      if (x > bv) {  // strict: equal values keep the lower column
        bv = x;
        bc = cbase + j;
      }
    }
    uint64_t key = ((uint64_t)key_of_f32(bv) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)bc);
    const uint64_t other = (uint64_t)__shfl_xor((long long)key, 32, 64);
    key = key > other ? key : other;
    if (half == 0) sKey[wc][wr * kLmWaveRows + i * 32 + row] = key;
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int r = t; r < kLmRows; r += 256)
    if (r0 + r < M) {
      const uint64_t a = sKey[0][r], b = sKey[1][r];
      part[(size_t)(r0 + r) * VT + vt] = a > b ? a : b;
    }
}

// One workgroup per request: wave w combines the vocabulary-tile partials of
// rows w, w + 4, ... (all 64 lanes load at once, 8 partials in flight per
// lane), then the first wave applies the greedy rule (accept while the draft
// equals the top choice; emit the top choice at the first mismatch, or the
// bonus after the last position).
__global__ __launch_bounds__(256) void k_lmhead_decide(const uint64_t *__restrict__ part,
                                                       const int32_t *__restrict__ tokens, int K,
                                                       int VT, int32_t *__restrict__ out_accepted,
                                                       int32_t *__restrict__ out_tokens,
                                                       int32_t *__restrict__ out_argmax) {
  __shared__ int s_am[64];
  const int b = blockIdx.x, t = threadIdx.x, l = t & 63, w = t >> 6;
  for (int p = w; p <= K; p += 4) {
    const uint64_t *pr = part + ((size_t)b * (K + 1) + p) * VT;
    uint64_t best = 0;
    for (int j0 = 0; j0 < VT; j0 += 64 * 8) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u * 64 + l;
        v[u] = j < VT ? pr[j] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) best = v[u] > best ? v[u] : best;
    }
    best = wave_max_u64(best);
    if (l == 0) s_am[p] = (int)(0xFFFFFFFFu - (uint32_t)best);
  }
  __syncthreads();
  if (w != 0) return;
  const int am = l <= K ? s_am[l] : -1;
  const int x = l < K ? tokens[(size_t)b * K + l] : -1;
  const uint64_t miss = __ballot(l < K && x != am);
  const int n = miss ? __builtin_ctzll(miss) : K;
  if (l <= K) {
    out_tokens[(size_t)b * (K + 1) + l] = l < n ? x : (l == n ? am : -1);
    if (out_argmax) out_argmax[(size_t)b * (K + 1) + l] = am;
  }
  if (l == 0) out_accepted[b] = n;
}

int lmhead_vocab_tiles(int V) { return (V + kLmCols - 1) / kLmCols; }

hipError_t launch_lmhead_greedy(const void *hidden, const void *weight, const int32_t *tokens,
                                int B, int K, int d, int V, int32_t *out_accepted,
                                int32_t *out_tokens, int32_t *out_argmax, uint64_t *part,
                                hipStream_t stream) {
  const int M = B * (K + 1);
  const int RT = (M + kLmRows - 1) / kLmRows;
  const int VT = lmhead_vocab_tiles(V);
  const int groups = (VT + 7) / 8;
  hipLaunchKernelGGL(k_lmhead_argmax, dim3(groups * 8 * RT), dim3(256), 0, stream,
                     (const u32x4 *)hidden, (const u32x4 *)weight, M, d, V, RT, VT, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_lmhead_decide, dim3(B), dim3(256), 0, stream, part, tokens, K, VT,
                     out_accepted, out_tokens, out_argmax);
  return hipGetLastError();
}

}  // namespace sv
