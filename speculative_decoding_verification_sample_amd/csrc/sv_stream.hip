// Greedy and merged-tree verification, one kernel each.  Every logit row is
// streamed once (argmax_tile); each tile publishes its key under the call's
// epoch tag, and the request's last tile (the last one dispatched) waits for
// the other tiles' tags, then decides with its first wave:
//  - greedy: accept drafts while each equals the target's top choice at its
//    position, emit the top choice at the first mismatch, or the bonus after
//    the last position (lotook.com explainer, four steps and FAQ; SubSpec
//    review on hip-studyrecord.tistory.com, Method part 2, verify step);
//  - tree: one wave64 per merged tree (N <= 64 nodes, one per lane); a node
//    matches when its token is the top choice at its parent and is accepted
//    when every node on its ancestor-mask row matches; the deepest accepted
//    node (lowest index on ties) ends the path (TAPS on aitrends.kr, section
//    "방법론": one target pass under an ancestor-preserving mask, the longest
//    accepted path is kept).
#include "sv_device.hpp"
#include "sv_kernels.hpp"
#include "sv_tiles.hpp"

namespace sv {

namespace {

// A row's top choice from its splits' keys; the keys are loaded eight at a
// time, all issued before any is compared (one round trip per eight).
__device__ __forceinline__ int combine_argmax(const uint64_t *part_key, size_t row, int S) {
  const uint64_t *pk = part_key + row * (size_t)S;
  uint64_t best = 0;
  for (int s0 = 0; s0 < S; s0 += 8) {
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = s0 + u < S ? load_agent(&pk[s0 + u]) : 0ull;
#pragma unroll
    for (int u = 0; u < 8; ++u) best = v[u] > best ? v[u] : best;
  }
  return (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
}

// Wave 0 of the last workgroup of request b.
__device__ void greedy_decide(const int32_t *tokens, int b, int K, int S,
                              const uint64_t *part_key, int32_t *out_accepted,
                              int32_t *out_tokens) {
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

// Wave 0 of the last workgroup of tree b.
__device__ void tree_decide(const int32_t *parents, const int32_t *node_tokens,
                            const uint8_t *anc_mask, int b, int N, int S,
                            const uint64_t *part_key, int32_t *out_path_len,
                            int32_t *out_path_nodes, int32_t *out_tokens) {
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
  // deepest accepted node, lowest index on ties (the root is always accepted)
  int key = accepted ? (depth << 8) | (255 - i) : -1;
  for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o, 64));
  const int best = key >= 0 ? 255 - (key & 255) : 0;
  const int d = key >= 0 ? max(0, key >> 8) : 0;
  const uint64_t path_bits = __shfl(anc, best, 64);
  const int a_best = __shfl(a, best, 64);
  // assemble in LDS (one wave: its LDS accesses stay in program order), then
  // one store per lane
  __shared__ int s_pn[64], s_ot[64];
  s_pn[i] = -1;
  s_ot[i] = i == d ? a_best : -1;
  __builtin_amdgcn_wave_barrier();
  // path nodes (root excluded) sit at position depth - 1
  if (node && i > 0 && ((path_bits >> i) & 1ull) && depth >= 1 && depth <= d) {
    s_pn[depth - 1] = i;
    s_ot[depth - 1] = tok;
  }
  __builtin_amdgcn_wave_barrier();
  if (node) {
    out_path_nodes[(size_t)b * N + i] = s_pn[i];
    out_tokens[(size_t)b * N + i] = s_ot[i];
  }
  if (i == 0) out_path_len[b] = d;
}

}  // namespace

// Greedy (rows_per_req = K + 1) or tree (rows_per_req = N) verify; one
// workgroup per (row, split), rows of a request consecutive.
template <int DT, bool TREE>
__global__ __launch_bounds__(kThreads) void k_argmax_fused(
    const char *__restrict__ target, int rows_per_req, int V, int S, u64 epoch,
    uint64_t *__restrict__ part_key, u64 *__restrict__ part_tag,
    const int32_t *__restrict__ tokens, const int32_t *__restrict__ parents,
    const uint8_t *__restrict__ anc_mask, int32_t *__restrict__ out_n,
    int32_t *__restrict__ out_nodes, int32_t *__restrict__ out_tokens) {
  const int row = blockIdx.x / S;
  const int s = blockIdx.x - row * S;
  const int b = row / rows_per_req;
  const int per_req = rows_per_req * S;
  const size_t row_bytes = (size_t)V * elem_bytes(DT);
  const uint64_t key = argmax_tile<DT>(target + (size_t)row * row_bytes, V, s);
  if (threadIdx.x == 0) {
    store_agent(&part_key[blockIdx.x], key);
    publish_tag(&part_tag[blockIdx.x], epoch);
  }
  if ((int)(blockIdx.x + 1) % per_req != 0) return;  // only the request's last tile decides
  __shared__ int s_flag;
  if (!block_wait_tags(part_tag + (size_t)b * per_req, per_req, epoch, &s_flag)) {
    if (threadIdx.x == 0) out_n[b] = -2;  // time-out: flag the request as failed
    return;
  }
  if (threadIdx.x >= 64) return;
  if (TREE)
    tree_decide(parents, tokens, anc_mask, b, rows_per_req, S, part_key, out_n, out_nodes,
                out_tokens);
  else
    greedy_decide(tokens, b, rows_per_req - 1, S, part_key, out_n, out_tokens);
}

hipError_t launch_greedy(const void *target, int dtype, const int32_t *tokens, int B, int K,
                         int V, int S, u64 epoch, uint64_t *part_key, u64 *part_tag,
                         int32_t *out_accepted, int32_t *out_tokens, hipStream_t stream) {
  dim3 grid(B * (K + 1) * S), block(kThreads);
  if (dtype == kBF16)
    hipLaunchKernelGGL((k_argmax_fused<kBF16, false>), grid, block, 0, stream,
                       (const char *)target, K + 1, V, S, epoch, part_key, part_tag, tokens,
                       nullptr, nullptr, out_accepted, nullptr, out_tokens);
  else
    hipLaunchKernelGGL((k_argmax_fused<kF32, false>), grid, block, 0, stream,
                       (const char *)target, K + 1, V, S, epoch, part_key, part_tag, tokens,
                       nullptr, nullptr, out_accepted, nullptr, out_tokens);
  return hipGetLastError();
}

hipError_t launch_tree(const void *target, int dtype, const int32_t *parents,
                       const int32_t *node_tokens, const uint8_t *anc_mask, int B, int N, int V,
                       int S, u64 epoch, uint64_t *part_key, u64 *part_tag, int32_t *out_path_len,
                       int32_t *out_path_nodes, int32_t *out_tokens, hipStream_t stream) {
  dim3 grid(B * N * S), block(kThreads);
  if (dtype == kBF16)
    hipLaunchKernelGGL((k_argmax_fused<kBF16, true>), grid, block, 0, stream,
                       (const char *)target, N, V, S, epoch, part_key, part_tag, node_tokens,
                       parents, anc_mask, out_path_len, out_path_nodes, out_tokens);
  else
    hipLaunchKernelGGL((k_argmax_fused<kF32, true>), grid, block, 0, stream,
                       (const char *)target, N, V, S, epoch, part_key, part_tag, node_tokens,
                       parents, anc_mask, out_path_len, out_path_nodes, out_tokens);
  return hipGetLastError();
}

}  // namespace sv
