// Two drafters' trees merged under one root, and the routing score of each
// (TAPS on aitrends.kr: "방법론", one target pass over both trees under an
// ancestor-preserving mask, the tree with the higher mean confidence
// preferred when only one is sent; "코드 예제", the merged block layout).
//
// One wave per request, one lane per merged node (N = n1 + n2 + 1 <= 64):
// node 0 = the shared root (tree 1's root token), nodes 1..n1 = tree 1's
// nodes with their parents, nodes n1+1..n1+n2 = tree 2's nodes (parent 0
// stays 0, parent p > 0 becomes p + n1).  A lane's ancestor set is found by
// walking up the merged parents (in LDS), and the wave writes the N x N
// mask one row per store.  The
// confidences are summed in node order by one lane in fp64, as the
// definition reads.
#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {

__global__ __launch_bounds__(64) void k_tree_merge(
    const int32_t *__restrict__ parents1, const int32_t *__restrict__ tokens1,
    const float *__restrict__ conf1, int n1, const int32_t *__restrict__ parents2,
    const int32_t *__restrict__ tokens2, const float *__restrict__ conf2, int n2,
    int32_t *__restrict__ out_parents, int32_t *__restrict__ out_tokens,
    uint8_t *__restrict__ out_mask, float *__restrict__ out_conf,
    int32_t *__restrict__ out_route) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int N = n1 + n2 + 1;
  const size_t o1 = (size_t)b * (n1 + 1), o2 = (size_t)b * (n2 + 1);
  // every input word this lane needs, loaded up front: node i of each tree
  const int a1 = i <= n1 ? parents1[o1 + i] : 0;
  const int a2 = i <= n2 ? parents2[o2 + i] : 0;
  const int k1 = i <= n1 ? tokens1[o1 + i] : 0;
  const int k2 = i <= n2 ? tokens2[o2 + i] : 0;
  const float c1 = i <= n1 ? conf1[o1 + i] : 0.f;
  const float c2 = i <= n2 ? conf2[o2 + i] : 0.f;
  // both input trees in BFS order: root -1, then 0 <= parent < node
  const bool bad1 = i <= n1 && (i == 0 ? a1 != -1 : (a1 < 0 || a1 >= i));
  const bool bad2 = i <= n2 && (i == 0 ? a2 != -1 : (a2 < 0 || a2 >= i));
  const bool valid = __ballot(bad1 || bad2) == 0;

  // merged node i: tree 1's node i, or tree 2's node i - n1 (fetched from
  // that lane)
  const int src = i <= n1 ? 0 : min(i - n1, 63);
  const int q = __shfl(a2, src, 64), kq = __shfl(k2, src, 64);
  int par = -1, tok = -1;
  if (i < N && valid) {
    par = i <= n1 ? a1 : (q == 0 ? 0 : q + n1);
    tok = i <= n1 ? k1 : kq;
  }
  __shared__ int s_par[64];
  __shared__ unsigned long long s_row[64];
  s_par[i] = par;
  __builtin_amdgcn_wave_barrier();
  unsigned long long row = 0;  // ancestors of node i and itself
  if (i < N && valid)
    for (int j = i; j >= 0; j = s_par[j]) row |= 1ull << j;
  s_row[i] = row;
  __builtin_amdgcn_wave_barrier();
  if (i < N) {
    out_parents[(size_t)b * N + i] = par;
    out_tokens[(size_t)b * N + i] = tok;
    // row by row: lane i writes column i (one coalesced byte store per row)
    uint8_t *m = out_mask + (size_t)b * N * N;
#pragma unroll 8
    for (int r = 0; r < N; ++r) m[(size_t)r * N + i] = (uint8_t)((s_row[r] >> i) & 1ull);
  }
  // lane 0 adds the confidences up in node order (lane reads)
  auto lane_f = [](float v, int j) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), j));
  };
  if (i == 0) {
    double m1 = 0.0, m2 = 0.0;
    if (valid) {
      double s1 = 0.0, s2 = 0.0;
      for (int j = 1; j <= n1; ++j) s1 += (double)lane_f(c1, j);
      for (int j = 1; j <= n2; ++j) s2 += (double)lane_f(c2, j);
      m1 = n1 > 0 ? s1 / n1 : 0.0;
      m2 = n2 > 0 ? s2 / n2 : 0.0;
    }
    if (out_conf) {
      out_conf[2 * b] = (float)m1;
      out_conf[2 * b + 1] = (float)m2;
    }
    if (out_route) out_route[b] = valid ? (m2 > m1 ? 1 : 0) : -1;
  }
}

hipError_t launch_tree_merge(const int32_t *parents1, const int32_t *tokens1, const float *conf1,
                             int n1, const int32_t *parents2, const int32_t *tokens2,
                             const float *conf2, int n2, int B, int32_t *out_parents,
                             int32_t *out_tokens, uint8_t *out_mask, float *out_conf,
                             int32_t *out_route, hipStream_t stream) {
  hipLaunchKernelGGL(k_tree_merge, dim3(B), dim3(64), 0, stream, parents1, tokens1, conf1, n1,
                     parents2, tokens2, conf2, n2, out_parents, out_tokens, out_mask, out_conf,
                     out_route);
  return hipGetLastError();
}

}  // namespace sv
