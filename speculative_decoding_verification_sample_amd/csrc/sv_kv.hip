// KV-cache commit after one speculative cycle.  The entries of rejected
// drafts are cut from the cache before the next cycle (lotook.com explainer,
// section on the KV cache); a drafter sharing the target's layers gets the
// target's values for the accepted entries (SubSpec review on
// hip-studyrecord.tistory.com, Method part 2, step 4 "Update KV"); a merged
// tree keeps its longest accepted path (TAPS on aitrends.kr, "방법론"), whose
// entries are gathered into consecutive slots.
//
// Cache [L][2][B][H][S][D], rows of D elements (bytes only are moved).
// Request b's cycle sits at slots c .. c+N-1 (c = cache_len[b]); after the
// commit slot c + j holds path element j (the root, then the path nodes by
// depth), j = 0 .. d, and new_len[b] = c + 1 + d.
//
// One workgroup per (layer, K/V, request), over its heads in passes of as
// many heads as its registers hold for this request's path.  Path node ids
// increase with depth and each is at least its depth, so a row can be the
// source of one move and the destination of another; each pass therefore
// reads every row it will move into registers, waits until all those loads
// have returned, and only then writes.  Different workgroups touch disjoint
// rows.
#include "sv_device.hpp"
#include "sv_kernels.hpp"

namespace sv {

namespace {
constexpr int kKvItemsPerThread = 8;  // 16-byte pieces held per lane
}

__global__ __launch_bounds__(kThreads) void k_kv_commit(
    char *__restrict__ kv, char *__restrict__ mirror, int B, int H, int S, size_t row_bytes,
    const int32_t *__restrict__ cache_len, const int32_t *__restrict__ path_len,
    const int32_t *__restrict__ path_nodes, int N, int32_t *__restrict__ new_len) {
  const int t = threadIdx.x;
  const int b = blockIdx.x % B;
  const int lk = blockIdx.x / B;  // layer * 2 + (0: K, 1: V)

  __shared__ int s_node[64];
  __shared__ int s_ok;
  // the path's node ids are loaded with its length, not after it (a lane
  // past the path ignores what it read)
  const int raw = path_nodes && t >= 1 && t <= N ? path_nodes[(size_t)b * N + t - 1] : t;
  const int c = cache_len[b];
  const int d = path_len[b];
  const bool dok = d >= 0 && d <= N - 1 && c >= 0 && (long)c + N <= S;
  if (t == 0) s_ok = dok;
  if (t < 64) s_node[t] = dok && t <= d ? (t == 0 ? 0 : raw) : -1;
  __syncthreads();
  // nodes strictly increasing, within the cycle's slots
  if (dok && t >= 1 && t <= d && (s_node[t] <= s_node[t - 1] || s_node[t] > N - 1)) s_ok = 0;
  __syncthreads();
  const bool ok = s_ok != 0;
  if (lk == 0 && t == 0) new_len[b] = ok ? c + 1 + d : -1;
  if (!ok) return;

  const int nch = (int)(row_bytes / 16);
  const int per_head = (d + 1) * nch;                       // 16-byte pieces of one head
  const int hp = max(1, (kKvItemsPerThread * kThreads) / per_head);  // heads per pass
  const size_t head_bytes = (size_t)S * row_bytes;
  const size_t base0 = ((size_t)lk * B + b) * H * head_bytes;
  for (int h0 = 0; h0 < H; h0 += hp) {
    const int items = min(hp, H - h0) * per_head;
    u32x4 buf[kKvItemsPerThread];
    // 1. read every row this pass moves
#pragma unroll
    for (int u = 0; u < kKvItemsPerThread; ++u) {
      const int i = t + u * kThreads;
      if (i < items) {
        const int ch = i % nch;
        const int rest = i / nch;
        const int j = rest % (d + 1);
        const int h = h0 + rest / (d + 1);
        const size_t off = base0 + h * head_bytes + (size_t)(c + s_node[j]) * row_bytes + ch * 16;
        buf[u] = *reinterpret_cast<const u32x4 *>(kv + off);
      }
    }
    // every load has returned before any lane of the workgroup writes
#pragma unroll
    for (int u = 0; u < kKvItemsPerThread; ++u)
      if (t + u * kThreads < items) asm volatile("" ::"v"(buf[u]));
    __syncthreads();
    // 2. write: the cache where the row moves, the mirror for every path row
#pragma unroll
    for (int u = 0; u < kKvItemsPerThread; ++u) {
      const int i = t + u * kThreads;
      if (i < items) {
        const int ch = i % nch;
        const int rest = i / nch;
        const int j = rest % (d + 1);
        const int h = h0 + rest / (d + 1);
        const size_t off = base0 + h * head_bytes + (size_t)(c + j) * row_bytes + ch * 16;
        if (s_node[j] != j) *reinterpret_cast<u32x4 *>(kv + off) = buf[u];
        if (mirror) *reinterpret_cast<u32x4 *>(mirror + off) = buf[u];
      }
    }
    // the next pass's reads come after this pass's writes (other heads: no
    // overlap, but keep the passes ordered)
    __syncthreads();
  }
}

hipError_t launch_kv_commit(void *kv, void *mirror, int L, int B, int H, int S, size_t row_bytes,
                            const int32_t *cache_len, const int32_t *path_len,
                            const int32_t *path_nodes, int N, int32_t *new_len,
                            hipStream_t stream) {
  dim3 grid((unsigned)L * 2u * (unsigned)B), block(kThreads);
  hipLaunchKernelGGL(k_kv_commit, grid, block, 0, stream, (char *)kv, (char *)mirror, B, H, S,
                     row_bytes, cache_len, path_len, path_nodes, N, new_len);
  return hipGetLastError();
}

int kv_items_per_wg() { return kKvItemsPerThread * kThreads; }

}  // namespace sv
