// The target's LM head fused in front of greedy verification: logits =
// hidden states x vocabulary matrix^T on the matrix cores, reduced to each
// row's top choice without ever writing the logits (lotook.com explainer,
// the four steps: one target pass yields the K+1 distributions, and the
// greedy rule of its FAQ accepts a draft only if it is the top choice).
//
// k_lmhead_argmax: one workgroup (4 waves) per 128-row x 256-column tile of
// the logits, d reduced in stages of 32 through double-buffered LDS with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation of exact bf16 products); the
// loads of the next three stages are in flight (in registers) while a stage
// is multiplied, to cover the memory latency with one workgroup per CU.
// Each wave owns 64 rows x 128 columns (2 x 4 blocks of 32 x 32).  LDS holds
// a stage as [k chunk of 8][row or column] 16-byte entries, so that the 32
// lanes reading one operand fragment touch 512 contiguous bytes.  The
// epilogue turns every logit into an order-preserving key (value, then the
// lowest column), takes the lane's best over its 4 column blocks, the best
// over the 32 lanes of a row by DPP moves, and the best of the two column
// waves in LDS: one 64-bit partial per (row, vocabulary tile).  The row
// tiles of one vocabulary tile run on the same XCD back to back, so that
// each slice of the vocabulary matrix comes from HBM once.
// k_lmhead_decide: one wave per request combines its rows' partials and
// applies the greedy rule.
#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLmRows = 128;   // rows per tile
constexpr int kLmCols = 256;   // vocabulary columns per tile
constexpr int kLmK = 32;       // d per LDS stage
constexpr int kLmChunks = kLmK / 8;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace

__global__ __launch_bounds__(256) void k_lmhead_argmax(const u32x4 *__restrict__ hidden,
                                                       const u32x4 *__restrict__ weight,
                                                       int M, int d, int V, int RT, int VT,
                                                       uint64_t *__restrict__ part) {
  // block -> (vocabulary tile vt, row tile rt): groups of 8 vocabulary tiles
  // times RT row tiles; the RT row tiles of one vocabulary tile share
  // blockIdx mod 8 (one XCD) and are dispatched within 8 RT blocks
  const int blk = blockIdx.x;
  const int grp = blk / (8 * RT), rem = blk - grp * 8 * RT;
  const int rt = rem >> 3, vt = grp * 8 + (rem & 7);
  if (vt >= VT) return;
  const int r0 = rt * kLmRows, v0 = vt * kLmCols;
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int wr = wv >> 1, wc = wv & 1;  // wave's 64-row and 128-column half
  const int dv = d >> 3;                // 16-byte chunks per row

  __shared__ u32x4 sA[2][kLmChunks][kLmRows];
  __shared__ u32x4 sB[2][kLmChunks][kLmCols];
  __shared__ uint64_t sKey[2][kLmRows];

  // staging: entry e = t + 256 j; A: 2 entries per thread, B: 4.  Rows at
  // or past M and columns at or past V load row M-1 / column V-1 instead
  // (unconditional loads keep the wait counts exact); their products only
  // reach rows that are never written and columns the epilogue drops.
  int a_row[2], a_c[2], b_col[4], b_c[4];
  const u32x4 *hrow[2], *wrow[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = t + 256 * j;
    a_row[j] = e >> 2;
    a_c[j] = e & 3;
    hrow[j] = hidden + (size_t)min(r0 + a_row[j], M - 1) * dv + a_c[j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = t + 256 * j;
    b_col[j] = e >> 2;
    b_c[j] = e & 3;
    wrow[j] = weight + (size_t)min(v0 + b_col[j], V - 1) * dv + b_c[j];
  }

  // three register sets of staged loads: stages s+1 .. s+3 are in flight
  // while stage s is multiplied out of LDS
  struct Stage {
    u32x4 a[2], b[4];
  };
  Stage R0, R1, R2;
  auto load_stage = [&](int s, Stage &R) {
    const int off = s * kLmChunks;
#pragma unroll
    for (int j = 0; j < 2; ++j) R.a[j] = hrow[j][off];
#pragma unroll
    for (int j = 0; j < 4; ++j) R.b[j] = __builtin_nontemporal_load(wrow[j] + off);
  };
  auto store_stage = [&](int buf, const Stage &R) {
#pragma unroll
    for (int j = 0; j < 2; ++j) sA[buf][a_c[j]][a_row[j]] = R.a[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) sB[buf][b_c[j]][b_col[j]] = R.b[j];
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][c][v] = 0.f;

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kLmK / 16; ++ks) {
      const int ch = ks * 2 + (l >> 5);
      bf16x8 fa[2], fb[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = as_bf16x8(sA[buf][ch][wr * 64 + i * 32 + (l & 31)]);
#pragma unroll
      for (int c = 0; c < 4; ++c) fb[c] = as_bf16x8(sB[buf][ch][wc * 128 + c * 32 + (l & 31)]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[c], acc[i][c], 0, 0, 0);
    }
  };
  // one stage: the set holding stage s was stored to LDS by the step before;
  // it now takes stage s + 3 (the last stage again near the end: loads stay
  // unconditional, so the waits before the LDS stores count exactly), stage
  // s is multiplied, and stage s + 1 is stored (past the end a copy of the
  // last stage lands in a buffer nothing reads)
  const int S = d / kLmK;
  auto step = [&](int s, Stage &cur, Stage &next) {
    load_stage(min(s + 3, S - 1), cur);
    compute(s & 1);
    store_stage((s + 1) & 1, next);
    __syncthreads();
  };
  load_stage(0, R0);
  load_stage(min(1, S - 1), R1);
  load_stage(min(2, S - 1), R2);
  store_stage(0, R0);
  __syncthreads();
  int s = 0;
  for (; s + 3 <= S; s += 3) {
    step(s, R0, R1);
    step(s + 1, R1, R2);
    step(s + 2, R2, R0);
  }
  if (s < S) step(s, R0, R1);
  if (s + 1 < S) step(s + 1, R1, R2);

  // epilogue: the best (value, lowest column) key of every row of the tile
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      uint64_t best = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = v0 + wc * 128 + c * 32 + (l & 31);
        const float x = col < V ? acc[i][c][v] : -INFINITY;
        const uint64_t key = ((uint64_t)key_of_f32(x) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)col);
        best = key > best ? key : best;
      }
      // best over the 32 lanes of this row (lanes l and l ^ 32 hold rows 4 apart)
      auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
      best = mx(best, dpp_u64<kDppXor1>(0, best));
      best = mx(best, dpp_u64<kDppXor2>(0, best));
      best = mx(best, dpp_u64<kDppHalfMirror>(0, best));
      best = mx(best, dpp_u64<kDppMirror>(0, best));
      best = mx(best, dpp_u64<kDppBcast15, 0xA>(0, best));
      if ((l & 31) == 31) {
        const int row = wr * 64 + i * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        sKey[wc][row] = best;
      }
    }
  }
  __syncthreads();
  if (t < kLmRows && r0 + t < M) {
    const uint64_t a = sKey[0][t], b = sKey[1][t];
    part[(size_t)(r0 + t) * VT + vt] = a > b ? a : b;
  }
}

// One wave per request: the top choice of each of its K+1 rows from the
// vocabulary-tile partials, then the greedy rule (accept while the draft
// equals the top choice; emit the top choice at the first mismatch, or the
// bonus after the last position).
__global__ __launch_bounds__(64) void k_lmhead_decide(const uint64_t *__restrict__ part,
                                                      const int32_t *__restrict__ tokens, int K,
                                                      int VT, int32_t *__restrict__ out_accepted,
                                                      int32_t *__restrict__ out_tokens,
                                                      int32_t *__restrict__ out_argmax) {
  const int b = blockIdx.x, l = threadIdx.x;
  int am = -1;
  for (int p = 0; p <= K; ++p) {
    const uint64_t *pr = part + ((size_t)b * (K + 1) + p) * VT;
    uint64_t best = 0;
    for (int j = l; j < VT; j += 64) best = pr[j] > best ? pr[j] : best;
    best = wave_max_u64(best);
    const int a = (int)(0xFFFFFFFFu - (uint32_t)best);
    if (l == p) am = a;
  }
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
  hipLaunchKernelGGL(k_lmhead_decide, dim3(B), dim3(64), 0, stream, part, tokens, K, VT,
                     out_accepted, out_tokens, out_argmax);
  return hipGetLastError();
}

}  // namespace sv
