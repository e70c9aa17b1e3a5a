// The target's LM head fused in front of greedy verification: logits =
// hidden states x vocabulary matrix^T on the matrix cores, reduced to each
// row's top choice without ever writing the logits (lotook.com explainer,
// the four steps: one target pass yields the K+1 distributions, and the
// greedy rule of its FAQ accepts a draft only if it is the top choice).
//
// k_lmhead_argmax: one workgroup (8 waves, two per SIMD) per 384-row x
// 256-column tile of the logits (all the rows of a verify call fit one
// tile, so the vocabulary matrix is read once), d reduced in stages of 64
// with v_mfma_f32_32x32x16_bf16 (fp32 accumulation of exact bf16 products).
// Each wave owns 96 rows x 128 columns (3 x 4 blocks of 32 x 32: 7
// fragment reads feed 12 products).  Operands
// go from global memory straight into two LDS stages of 80 KB (loads that
// write LDS, no register staging): while one stage is multiplied the next
// arrives.  A stage holds each row's 128 bytes of d (eight 16-byte chunks,
// one whole cache line, fetched by 8 lanes of one load) side by side, the
// chunk position XOR-ed with bits 1..3 of the row, so that the 16 lanes of
// a fragment read quarter touch 16 different bank groups.  The wide tile
// halves the re-reads of the hidden states (every tile reads all of them).
// k_lmhead_decide: one workgroup per request combines its rows' partials and
// applies the greedy rule.
#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLmRows = 384;   // rows per tile (12 blocks of 32)
constexpr int kLmCols = 256;   // vocabulary columns per tile (8 blocks of 32)
constexpr int kLmThreads = 512;
constexpr int kLmK = 64;       // d per LDS stage
constexpr int kLmChunks = kLmK / 8;                // 16-byte chunks per row and stage
constexpr int kLmWaveRows = kLmRows / 4;           // each wave: 96 rows x 128 columns
constexpr int kLmWaveCols = kLmCols / 2;
constexpr int kLmRB = kLmWaveRows / 32;            // 3 row blocks per wave
constexpr int kLmCB = kLmWaveCols / 32;            // 4 column blocks per wave
constexpr int kLmColWaves = kLmCols / kLmWaveCols; // waves across the columns
constexpr int kLmEntA = kLmRows * kLmChunks;       // 3072 entries of 16 bytes
constexpr int kLmEnt = kLmEntA + kLmCols * kLmChunks;  // 5120 entries: 80 KB a stage
constexpr int kLmLoadsA = kLmEntA / kLmThreads;    // 6 wave loads of 1 KB per wave
constexpr int kLmLoadsB = kLmCols * kLmChunks / kLmThreads;  // 4

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// slot of chunk c of row (or column) r within its operand's part of a stage
__device__ __forceinline__ int lm_entry(int r, int c) { return r * kLmChunks + (c ^ ((r >> 1) & 7)); }

typedef __attribute__((address_space(3))) void *lds_ptr;

}  // namespace

__global__ __launch_bounds__(kLmThreads) void k_lmhead_argmax(const u32x4 *__restrict__ hidden,
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
  const int wr = wv / kLmColWaves, wc = wv % kLmColWaves;  // wave's rows and columns

  __shared__ u32x4 ring[2 * kLmEnt];

  // Loads: wave wv fills entries (wv * n + j) * 64 .. + 64 of each operand
  // part, lane l entry + l: row e / 8 (8 lanes read its 128 bytes) and the
  // chunk its slot holds.  Rows at or past M and columns at or past V load
  // row M-1 / column V-1; their products only reach rows that are never
  // written and columns the epilogue drops.
  uint32_t oa[kLmLoadsA], ob[kLmLoadsB];  // byte offsets from the tile's first row / column
#pragma unroll
  for (int j = 0; j < kLmLoadsA; ++j) {
    const int e = (wv * kLmLoadsA + j) * 64 + l, r = e >> 3;
    const int c = (e & 7) ^ ((r >> 1) & 7);
    oa[j] = (uint32_t)((min(r0 + r, M - 1) - r0) * d + c * 8) * 2u;
  }
#pragma unroll
  for (int j = 0; j < kLmLoadsB; ++j) {
    const int e = (wv * kLmLoadsB + j) * 64 + l, r = e >> 3;
    const int c = (e & 7) ^ ((r >> 1) & 7);
    ob[j] = (uint32_t)((min(v0 + r, V - 1) - v0) * d + c * 8) * 2u;
  }
  // buffer descriptors over the tile's rows / columns (32-bit lane offsets,
  // the stage's offset in a scalar register)
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(reinterpret_cast<const char *>(hidden) + (size_t)r0 * d * 2), (short)0,
      (int)((size_t)(min(M - r0, kLmRows)) * d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(reinterpret_cast<const char *>(weight) + (size_t)v0 * d * 2), (short)0,
      (int)((size_t)(min(V - v0, kLmCols)) * d * 2), 0x00020000);
  // stage src (d from 64 src) into ring slot `slot`; 10 loads per wave
  auto issue = [&](int slot, int src) {
    u32x4 *base = ring + slot * kLmEnt;
    const int so = src * (kLmK * 2);
#pragma unroll
    for (int j = 0; j < kLmLoadsA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr)(base + (wv * kLmLoadsA + j) * 64), 16,
                                               oa[j], so, 0, 0);
#pragma unroll
    for (int j = 0; j < kLmLoadsB; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr)(base + kLmEntA + (wv * kLmLoadsB + j) * 64),
                                               16, ob[j], so, 0, 2 /* nontemporal: read once */);
  };

  f32x16 acc[kLmRB][kLmCB];
#pragma unroll
  for (int i = 0; i < kLmRB; ++i)
#pragma unroll
    for (int c = 0; c < kLmCB; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][c][v] = 0.f;

  // fragments of k-step ks (16 of d) of slot `slot`, and their 12 products
  auto read_frags = [&](int slot, int ks, bf16x8 (&fa)[kLmRB], bf16x8 (&fb)[kLmCB]) {
    const u32x4 *base = ring + slot * kLmEnt;
    const int ch = ks * 2 + (l >> 5);
#pragma unroll
    for (int i = 0; i < kLmRB; ++i)
      fa[i] = as_bf16x8(base[lm_entry(wr * kLmWaveRows + i * 32 + (l & 31), ch)]);
#pragma unroll
    for (int c = 0; c < kLmCB; ++c)
      fb[c] = as_bf16x8(base[kLmEntA + lm_entry(wc * kLmWaveCols + c * 32 + (l & 31), ch)]);
  };
  auto mma = [&](const bf16x8 (&fa)[kLmRB], const bf16x8 (&fb)[kLmCB]) {
#pragma unroll
    for (int i = 0; i < kLmRB; ++i)
#pragma unroll
      for (int c = 0; c < kLmCB; ++c)
        acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[c], acc[i][c], 0, 0, 0);
  };

  // Step s: wait until this wave's loads of stage s have landed (nothing
  // else is outstanding); the barrier makes every wave's part visible and
  // guarantees every wave is done with stage s - 1, whose slot then takes
  // stage s + 1 (past the end, a copy of the last stage into a slot nothing
  // reads any more).  The accumulators take 192 of a wave's 256 registers,
  // so a k-step's fragments are read just before its products; the other
  // wave on the SIMD runs its products meanwhile.
  const int S = d / kLmK;
  issue(0, 0);
  for (int s = 0; s < S; ++s) {
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    issue((s + 1) & 1, min(s + 1, S - 1));
    const int slot = s & 1;
#pragma unroll
    for (int ks = 0; ks < kLmK / 16; ++ks) {
      bf16x8 fa[kLmRB], fb[kLmCB];
      read_frags(slot, ks, fa, fb);
      mma(fa, fb);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the ring is idle
  __builtin_amdgcn_s_barrier();

  // epilogue: each row's best (value, lowest column).  Per row block the
  // wave writes its 32 x 128 logits to LDS (the ring is free now), then lane
  // l scans columns 64 (l / 32) .. + 64 of row l % 32, and the two halves
  // combine through one lane exchange.
  constexpr int kT = kLmWaveCols + 1;  // transpose row stride (floats)
  float *sT = reinterpret_cast<float *>(ring) + wv * (32 * kT);
  uint64_t(*sKey)[kLmRows] =
      reinterpret_cast<uint64_t(*)[kLmRows]>(reinterpret_cast<float *>(ring) + 8 * 32 * kT);
#pragma unroll
  for (int i = 0; i < kLmRB; ++i) {
#pragma unroll
    for (int c = 0; c < kLmCB; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        sT[row * kT + c * 32 + (l & 31)] = acc[i][c][v];
      }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const int row = l & 31, half = l >> 5;
    constexpr int kHalf = kLmWaveCols / 2;
    const int cbase = v0 + wc * kLmWaveCols + half * kHalf;
    float bv = -INFINITY;
    int bc = 0x7FFFFFFF;
    for (int j = 0; j < kHalf; ++j) {
      const float x = cbase + j < V ? sT[row * kT + half * kHalf + j] : -INFINITY;
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
  for (int r = t; r < kLmRows; r += kLmThreads)
    if (r0 + r < M) {
      uint64_t a = sKey[0][r];
#pragma unroll
      for (int q = 1; q < kLmColWaves; ++q) a = sKey[q][r] > a ? sKey[q][r] : a;
      part[(size_t)(r0 + r) * VT + vt] = a;
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
  hipLaunchKernelGGL(k_lmhead_argmax, dim3(groups * 8 * RT), dim3(kLmThreads), 0, stream,
                     (const u32x4 *)hidden, (const u32x4 *)weight, M, d, V, RT, VT, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_lmhead_decide, dim3(B), dim3(256), 0, stream, part, tokens, K, VT,
                     out_accepted, out_tokens, out_argmax);
  return hipGetLastError();
}

}  // namespace sv
