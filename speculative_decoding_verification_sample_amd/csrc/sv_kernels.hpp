// Host-side launchers of the verify kernels (internal to libspecverify.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_layout.hpp"

namespace sv {

// greedy / merged-tree verify, one kernel each (sv_stream.hip)
hipError_t launch_greedy(const void *target, int dtype, const int32_t *tokens, int B, int K,
                         int V, int S, u64 epoch, uint64_t *part_key, u64 *part_tag,
                         int32_t *out_accepted, int32_t *out_tokens, hipStream_t stream);
hipError_t launch_tree(const void *target, int dtype, const int32_t *parents,
                       const int32_t *node_tokens, const uint8_t *anc_mask, int B, int N, int V,
                       int S, u64 epoch, uint64_t *part_key, u64 *part_tag, int32_t *out_path_len,
                       int32_t *out_path_nodes, int32_t *out_tokens, hipStream_t stream);

// sampling verify (sv_sample.hip); phase 0 = whole call in one kernel,
// 1 = streaming tiles only, 2 = residual tiles only (around the top-p kernel)
hipError_t launch_sample(const SampleArgs &args, int dtype, hipStream_t stream);

// the ratio tests of a top-p call with batch-wide parameters, once per
// request, after the nucleus launches (sv_sample.hip)
hipError_t launch_topp_decide(const SampleArgs &args, hipStream_t stream);
// ... then the residual masses of the drawn row pairs and the draw, in two
// launches that never wait on each other's workgroups (sv_sample.hip)
hipError_t launch_topp_residual(const SampleArgs &args, int dtype, hipStream_t stream);

// workgroups of the fused sampling kernel resident at once (cached per dtype)
int resident_workgroups(int dtype);

// top-p nucleus threshold per row (sv_topp.hip)
hipError_t launch_topp_select(const SampleArgs &args, int dtype, hipStream_t stream);

// two trees merged under one root, with confidence routing (sv_merge.hip)
hipError_t launch_tree_merge(const int32_t *parents1, const int32_t *tokens1, const float *conf1,
                             int n1, const int32_t *parents2, const int32_t *tokens2,
                             const float *conf2, int n2, int B, int32_t *out_parents,
                             int32_t *out_tokens, uint8_t *out_mask, float *out_conf,
                             int32_t *out_route, hipStream_t stream);

// LM head fused with greedy verification (sv_lmhead.hip)
int lmhead_vocab_tiles(int V);
hipError_t launch_lmhead_greedy(const void *hidden, const void *weight, const int32_t *tokens,
                                int B, int K, int d, int V, int32_t *out_accepted,
                                int32_t *out_tokens, int32_t *out_argmax, uint64_t *part,
                                hipStream_t stream);

// KV-cache commit after a cycle (sv_kv.hip)
hipError_t launch_kv_commit(void *kv, void *mirror, int L, int B, int H, int S, size_t row_bytes,
                            const int32_t *cache_len, const int32_t *path_len,
                            const int32_t *path_nodes, int N, int32_t *new_len,
                            hipStream_t stream);
// 16-byte pieces one commit workgroup holds at once
int kv_items_per_wg();

}  // namespace sv
