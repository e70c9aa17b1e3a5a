// Temperature-0 decisions after the argmax streaming pass.
//  - k_greedy_decide: one wave64 per request; lane i holds the target's top
//    choice a_i at position i; a ballot of (draft_i == a_i) gives the first
//    mismatch n; emit the drafts before it and a_n (the replacement, or the
//    bonus when every draft matched).  Greedy accepts only the target's top
//    choice (lotook.com explainer, FAQ on losslessness; SubSpec review on
//    hip-studyrecord.tistory.com, Method part 2, verify step).
//  - k_tree_decide: one wave64 per merged tree (N <= 64 nodes, one per
//    lane).  A node matches when its token is the top choice at its parent;
//    it is accepted when every node on its ancestor-mask row matches; the
//    deepest accepted node (lowest index on ties) ends the path, which is
//    read off that node's mask row (TAPS on aitrends.kr, section "방법론":
//    an ancestor-preserving mask lets one target pass check every path, and
//    the longest accepted path is kept).
#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {

namespace {

__device__ __forceinline__ int combine_argmax(const uint64_t *part_key, size_t row, int S) {
  const uint64_t *pk = part_key + row * (size_t)S;
  uint64_t best = 0;
  for (int s = 0; s < S; ++s) best = pk[s] > best ? pk[s] : best;
  return (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
}

}  // namespace

__global__ __launch_bounds__(64) void k_greedy_decide(
    const int32_t *__restrict__ tokens, int K, int S, const uint64_t *__restrict__ part_key,
    int32_t *__restrict__ out_accepted, int32_t *__restrict__ out_tokens) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  int a = -1, x = -1;
  if (i <= K) a = combine_argmax(part_key, (size_t)b * (K + 1) + i, S);
  if (i < K) x = tokens[(size_t)b * K + i];
  const bool match = i < K && x == a;
  const uint64_t m = __ballot(match);
  const uint64_t live = K >= 64 ? ~0ull : ((1ull << K) - 1ull);
  const uint64_t miss = ~m & live;
  const int n = miss ? __builtin_ctzll(miss) : K;
  if (i <= K) out_tokens[(size_t)b * (K + 1) + i] = i < n ? x : (i == n ? a : -1);
  if (i == 0) out_accepted[b] = n;
}

__global__ __launch_bounds__(64) void k_tree_decide(
    const int32_t *__restrict__ parents, const int32_t *__restrict__ node_tokens,
    const uint8_t *__restrict__ anc_mask, int N, int S, const uint64_t *__restrict__ part_key,
    int32_t *__restrict__ out_path_len, int32_t *__restrict__ out_path_nodes,
    int32_t *__restrict__ out_tokens) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool node = i < N;
  int a = -1, par = -1, tok = -1;
  uint64_t anc = 0;
  if (node) {
    a = combine_argmax(part_key, (size_t)b * N + i, S);
    par = parents[(size_t)b * N + i];
    tok = node_tokens[(size_t)b * N + i];
    const uint8_t *mrow = anc_mask + ((size_t)b * N + i) * (size_t)N;
    for (int j = 0; j < N; ++j)
      if (mrow[j]) anc |= 1ull << j;
  }
  // the parent's top choice, fetched from the parent's lane
  const int src = (par >= 0 && par < N) ? par : i;
  const int a_par = __shfl(a, src, 64);
  const bool match = node && (i == 0 || (par >= 0 && par < N && tok == a_par));
  const uint64_t match_bits = __ballot(match);
  const bool accepted = node && (anc & ~match_bits) == 0;
  const int depth = node ? __popcll(anc) - 1 : -1;
  // deepest accepted node, lowest index on ties (root is always accepted)
  int key = accepted ? (depth << 8) | (255 - i) : -1;
  for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o, 64));
  const int best = key >= 0 ? 255 - (key & 255) : 0;
  const int d = key >= 0 ? max(0, key >> 8) : 0;
  const uint64_t path_bits = __shfl(anc, best, 64);
  const int a_best = __shfl(a, best, 64);
  // assemble the outputs in LDS, then one coalesced store per lane
  __shared__ int s_pn[64], s_ot[64];
  s_pn[i] = -1;
  s_ot[i] = i == d ? a_best : -1;
  __syncthreads();
  // path nodes (root excluded) sit at position depth - 1
  if (node && i > 0 && ((path_bits >> i) & 1ull) && depth >= 1 && depth <= d)
    s_pn[depth - 1] = i, s_ot[depth - 1] = tok;
  __syncthreads();
  if (node) {
    out_path_nodes[(size_t)b * N + i] = s_pn[i];
    out_tokens[(size_t)b * N + i] = s_ot[i];
  }
  if (i == 0) out_path_len[b] = d;
}

hipError_t launch_greedy_decide(const int32_t *tokens, int B, int K, int S,
                                const uint64_t *part_key, int32_t *out_accepted,
                                int32_t *out_tokens, hipStream_t stream) {
  hipLaunchKernelGGL(k_greedy_decide, dim3(B), dim3(64), 0, stream, tokens, K, S, part_key,
                     out_accepted, out_tokens);
  return hipGetLastError();
}

hipError_t launch_tree_decide(const int32_t *parents, const int32_t *node_tokens,
                              const uint8_t *anc_mask, int B, int N, int S,
                              const uint64_t *part_key, int32_t *out_path_len,
                              int32_t *out_path_nodes, int32_t *out_tokens,
                              hipStream_t stream) {
  hipLaunchKernelGGL(k_tree_decide, dim3(B), dim3(64), 0, stream, parents, node_tokens,
                     anc_mask, N, S, part_key, out_path_len, out_path_nodes, out_tokens);
  return hipGetLastError();
}

}  // namespace sv
