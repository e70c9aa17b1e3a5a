/*
 * spec_verify.h — C ABI of the MI355X (gfx950) speculative-decoding verify
 * library (libspecverify.so).
 *
 * The operation (p = target distribution, q = draft distribution):
 *  - one speculative cycle drafts K tokens with their draft distributions, then
 *    one target pass yields K+1 target distributions; the drafts are checked
 *    left to right, the first rejected one and everything after it is
 *    dropped, a replacement is drawn at the rejection, or a bonus token from
 *    the (K+1)-th distribution when every draft survives
 *    (lotook.com "What is speculative decoding?", section "단계별로 어떻게
 *    작동할까요", the four steps of a cycle);
 *  - a draft x ~ q is accepted with probability min(1, p(x)/q(x)); after a
 *    rejection the replacement is drawn from normalize(max(0, p - q));
 *    temperature and top-p are applied to p and q before the test
 *    (ariser.io "Speculative Decoding: 작은 모델이 먼저 쓰면 큰 모델도
 *    빨라진다", section "같은 분포를 지키는 작은 장치");
 *  - at temperature 0 a draft is accepted only if it is the target's top
 *    choice (lotook.com, FAQ on losslessness; SubSpec review on
 *    hip-studyrecord.tistory.com, Method part 2, verify step);
 *  - two drafters' trees merged under one root are verified in one target
 *    pass under an ancestor mask, keeping the longest accepted path
 *    (aitrends.kr "TAPS: 추측 샘플링을 위한 작업 인지형 제안 분포 연구",
 *    sections "방법론" and "코드 예제").
 *
 * Readings where the pages leave a step open:
 *  - accept iff u * q'(x) < p'(x), u in [0, 1) per position (u_accept[b, i]);
 *  - one uniform per request (u_sample[b]) draws the replacement or bonus by
 *    inverse CDF over ascending vocabulary ids: the smallest j with
 *    sum_{k<=j} r_k > u * S, S = sum_k r_k;
 *  - top-p: after temperature, keep the largest logits, whole tie groups,
 *    until the tempered mass first reaches top_p, renormalise; top_p = 1 is off;
 *  - argmax ties resolve to the lowest vocabulary id; -0.0 equals +0.0;
 *  - a draft token outside [0, V) is rejected (sampling) / a mismatch (greedy);
 *  - tree: a child is checked against the target's top choice at its parent;
 *    the deepest accepted node wins, the lowest node index on ties.
 *
 * Conventions shared by every entry point:
 *  - Device pointers live on the current HIP device; host scalars are passed
 *    by value.  Logit tensors are dense row-major; bf16 tensors hold raw
 *    16-bit patterns.  Each logit row must hold at least one finite value
 *    (-inf entries are allowed and have probability 0; NaN / +inf are not).
 *  - The caller owns every buffer.  The library never allocates or frees
 *    device memory and keeps no state between calls (outside the optional
 *    profiling hook below, and the one array per GPU that the loader places
 *    in device memory for spec_verify_sample_noalloc).  Inputs are read-only.
 *  - `workspace` is caller-provided device scratch of at least
 *    spec_verify_workspace_bytes(...) bytes, 256-byte aligned.  It needs no
 *    clearing: every call tags what it writes there with fresh epoch bits.
 *    Its contents are undefined after the call and it must not be shared by
 *    calls that may run concurrently.
 *  - Workgroups of one call hand partial results to each other through the
 *    workspace and wait for them with a bounded spin.  Should such a wait
 *    ever run out (it waits only on workgroups already dispatched, so it
 *    should not), the request's out_accepted / out_path_len is set to -2.
 *  - Calls validate every argument on the host first; on any failure they
 *    return a negative SPEC_ERR_* code and enqueue nothing.  On success they
 *    enqueue kernels on `stream` and return SPEC_OK without synchronising;
 *    outputs are valid once the stream has completed.  A failed kernel
 *    launch returns SPEC_ERR_HIP.
 *  - Limits: B >= 1; 1 <= K <= 63 (sample, greedy); 1 <= N <= 64 (tree);
 *    1 <= V <= 2^31 - 1 and B * rows * V addressable.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

enum {
  SPEC_OK = 0,
  SPEC_ERR_NULL = -1,      /* a required pointer is NULL */
  SPEC_ERR_SHAPE = -2,     /* B, K, N or V out of range */
  SPEC_ERR_PARAM = -3,     /* temperature not finite / <= 0, top_p not in (0, 1], bad dtype, op or element size */
  SPEC_ERR_WORKSPACE = -4, /* workspace smaller than spec_verify_workspace_bytes() */
  SPEC_ERR_ALIGN = -5,     /* workspace not 256-byte aligned, logits not element aligned, or a cache row / base not 16-byte aligned */
  SPEC_ERR_HIP = -6        /* a HIP launch or runtime call failed */
};

enum { SPEC_OP_GREEDY = 0, SPEC_OP_SAMPLE = 1, SPEC_OP_TREE = 2 };

/* Bytes of workspace a call with these sizes needs (host only, pure).
 * op: SPEC_OP_*; K_or_N: K for greedy/sample, N for tree; use_top_p: nonzero
 * if the sampling call will pass top_p < 1.  Returns 0 for invalid sizes. */
size_t spec_verify_workspace_bytes(int op, int B, int K_or_N, int V, int dtype,
                                   int use_top_p);

/* Greedy (temperature-0) verify of B requests.
 *   target_logits [B, K+1, V] (dtype), draft_tokens [B, K] int32.
 *   out_accepted [B]: n = number of leading drafts equal to the target's top
 *     choice at their position;
 *   out_tokens [B, K+1]: drafts 0..n-1, then the target's top choice at
 *     position n (the replacement, or the bonus when n == K), then -1. */
int spec_verify_greedy(const void *target_logits, int dtype,
                       const int32_t *draft_tokens, int B, int K, int V,
                       int32_t *out_accepted, int32_t *out_tokens,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Sampling verify of B requests at a batch-wide temperature and top-p.
 *   target_logits [B, K+1, V], draft_logits [B, K, V] (same dtype),
 *   draft_tokens [B, K] int32, u_accept [B, K] and u_sample [B] float32 in
 *   [0, 1); temperature > 0 and finite; top_p in (0, 1], 1 = off.
 *   out_accepted [B], out_tokens [B, K+1] as in the greedy call, with the
 *   replacement drawn from normalize(max(0, p' - q')) at the first
 *   rejection, or the bonus from p'_K;
 *   optional (may be NULL): out_p_draft / out_q_draft [B, K] = p'_i(x_i),
 *   q'_i(x_i) for every position; out_residual_mass [B] = S, the mass the
 *   replacement (or bonus) was drawn from. */
int spec_verify_sample(const void *target_logits, const void *draft_logits, int dtype,
                       const int32_t *draft_tokens, const float *u_accept,
                       const float *u_sample, float temperature, float top_p,
                       int B, int K, int V, int32_t *out_accepted, int32_t *out_tokens,
                       float *out_p_draft, float *out_q_draft, float *out_residual_mass,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* spec_verify_sample on a workspace the library holds, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Arguments, outputs and errors as
 * spec_verify_sample, without workspace / workspace_bytes.  The workspace is
 * one array of SPEC_SCRATCH_BYTES in device memory per GPU, held until the
 * process ends; calls needing more (spec_verify_workspace_bytes(
 * SPEC_OP_SAMPLE, ...) > SPEC_SCRATCH_BYTES) return SPEC_ERR_WORKSPACE with
 * nothing enqueued.  The call allocates nothing.  Every call on one GPU uses
 * that GPU's array: calls that may overlap on one GPU (other streams, other
 * threads) race and must not be issued; calls in one stream are ordered and
 * safe.  Nothing in the array needs clearing between calls (each call tags
 * what it writes with fresh epoch bits).  The first call on a device looks
 * up the array's address on that device (SPEC_ERR_HIP if that fails). */
#define SPEC_SCRATCH_BYTES (32u << 20)
int spec_verify_sample_noalloc(const void *target_logits, const void *draft_logits, int dtype,
                               const int32_t *draft_tokens, const float *u_accept,
                               const float *u_sample, float temperature, float top_p, int B,
                               int K, int V, int32_t *out_accepted, int32_t *out_tokens,
                               float *out_p_draft, float *out_q_draft,
                               float *out_residual_mass, hipStream_t stream);

/* Sampling verify with per-request temperature and top-p, greedy and
 * sampling requests mixed in one batch (temperature 0 is the greedy rule:
 * accept a draft only if it is the target's top choice; lotook.com
 * explainer, FAQ; the sampling rule and its settings as in
 * spec_verify_sample).
 *   Arguments as spec_verify_sample, except: temperature [B] float32 on the
 *   device (0 = greedy for that request, else > 0 and finite); top_p [B]
 *   float32 on the device, each in (0, 1], or NULL for 1 everywhere.
 *   A greedy request reads only its target rows (its draft rows, u_accept
 *   and u_sample are ignored); its out_p_draft / out_q_draft /
 *   out_residual_mass entries are 0.  A request whose temperature or top_p
 *   is out of range gets out_accepted = -3 and out_tokens = -1.
 *   Workspace: spec_verify_workspace_bytes(SPEC_OP_SAMPLE, ..., use_top_p)
 *   with use_top_p nonzero when top_p is not NULL. */
int spec_verify_mixed(const void *target_logits, const void *draft_logits, int dtype,
                      const int32_t *draft_tokens, const float *u_accept,
                      const float *u_sample, const float *temperature, const float *top_p,
                      int B, int K, int V, int32_t *out_accepted, int32_t *out_tokens,
                      float *out_p_draft, float *out_q_draft, float *out_residual_mass,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Greedy verify of B merged draft trees of N nodes each.
 *   target_logits [B, N, V]: row i = the target's next-token logits after
 *     the path root..i; parents [B, N] int32 (parents[0] = -1, 0 <= parents[i] < i);
 *   node_tokens [B, N] int32; anc_mask [B, N, N] uint8, nonzero = ancestor-or-self.
 *   The GPU trusts that anc_mask is the ancestor closure of parents (it never
 *   indexes out of range if it is not, but the result is then unspecified).
 *   out_path_len [B]: d = depth of the deepest accepted node;
 *   out_path_nodes [B, N]: node ids of the accepted path (root excluded, by
 *     depth), then -1;
 *   out_tokens [B, N]: the path's tokens, then the target's top choice after
 *     the last path node, then -1. */
int spec_verify_tree(const void *target_logits, int dtype, const int32_t *parents,
                     const int32_t *node_tokens, const uint8_t *anc_mask, int B, int N,
                     int V, int32_t *out_path_len, int32_t *out_path_nodes,
                     int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* The target's LM head fused in front of greedy verification: the logits
 * l[r][v] = sum_k hidden[r][k] * weight[v][k] of the K+1 target positions
 * are formed on the matrix cores and reduced straight to each row's top
 * choice; they are never written to memory (lotook.com explainer, the four
 * steps: one target pass yields the K+1 distributions; FAQ: greedy accepts a
 * draft only if it is the top choice).
 *   hidden [B, K+1, d] bf16 (the target's final hidden states), weight
 *   [V, d] bf16 (the vocabulary matrix, one row per token), both row-major
 *   and 16-byte aligned; d a multiple of 64; 1 <= K <= 63.
 *   Products of bf16 values are exact and accumulate in fp32 (the order of
 *   accumulation is not specified); ties in a row go to the lowest id.
 *   out_accepted [B], out_tokens [B, K+1] as spec_verify_greedy;
 *   out_argmax [B, K+1] int32 or NULL: each row's top choice.
 *   workspace: spec_lmhead_workspace_bytes() bytes, 256-byte aligned, no
 *   clearing needed.  Two launches on `stream`. */
size_t spec_lmhead_workspace_bytes(int B, int K, int d, int V);
int spec_lmhead_greedy(const void *hidden, const void *weight, const int32_t *draft_tokens, int B,
                       int K, int d, int V, int32_t *out_accepted, int32_t *out_tokens,
                       int32_t *out_argmax, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Two drafters' trees merged under one root for one target pass, with the
 * routing score of each tree (TAPS, "방법론": merged-tree verification
 * under an ancestor-preserving mask, the tree with the higher mean
 * confidence preferred when one is sent; "코드 예제": the merged layout).
 *   parents_t [B, n_t + 1] int32 (BFS order: node 0 the root with parent -1,
 *   0 <= parent[i] < i), tokens_t [B, n_t + 1] int32, conf_t [B, n_t + 1]
 *   float32 (the drafter's probability of each node's token; the root's is
 *   not used), t = 1, 2; n1 + n2 + 1 = N <= 64.
 *   out_parents / out_tokens [B, N], out_mask [B, N, N] uint8: node 0 = the
 *   shared root (tree 1's token), nodes 1..n1 = tree 1's, n1+1..N-1 = tree
 *   2's non-root nodes (parent 0 stays 0, parent p > 0 becomes p + n1); mask
 *   row i = the ancestors of node i and itself.  These are the inputs of
 *   spec_verify_tree.
 *   out_conf [B, 2] float32 or NULL: mean conf over each tree's non-root
 *   nodes (0 for an empty tree); out_route [B] int32 or NULL: 1 if tree 2's
 *   mean is larger, else 0.  A request with an invalid tree gets route -1,
 *   parents and tokens -1 and a zero mask. */
int spec_tree_merge(const int32_t *parents1, const int32_t *tokens1, const float *conf1, int n1,
                    const int32_t *parents2, const int32_t *tokens2, const float *conf2, int n2,
                    int B, int32_t *out_parents, int32_t *out_tokens, uint8_t *out_mask,
                    float *out_conf, int32_t *out_route, hipStream_t stream);

/* KV-cache commit after one cycle (next to the verify: the entries of
 * rejected drafts are cut away; lotook.com explainer, section on the KV
 * cache; a drafter sharing the target's layers receives the target's entries,
 * SubSpec review, Method part 2, step 4; a merged tree keeps its longest
 * accepted path, TAPS, "방법론").
 *   kv [L, 2, B, H, S, D] device buffer, elements of elem_bytes (1, 2, 4 or
 *     8; only bytes are moved), D * elem_bytes a multiple of 16, 16-byte
 *     aligned.  Request b's cycle wrote its N entries at slots c .. c+N-1,
 *     c = cache_len[b]: slot c + i holds tree node i (or linear position i);
 *     node 0 is the root (the token emitted by the previous cycle).
 *   path_len [B] = d (out_path_len of spec_verify_tree, or out_accepted of
 *     the linear calls); path_nodes [B, N] (out_path_nodes of
 *     spec_verify_tree), or NULL for a linear draft (positions 1 .. d).
 *   After the call slot c + j holds path element j (j = 0 .. d: the root,
 *   then the path by depth); other slots are unchanged; new_len[b] =
 *   c + 1 + d.  mirror (NULL or a second cache of the same layout, not kv)
 *   receives the same d + 1 entries at the same slots.
 *   A request with d outside [0, N-1], c < 0, c + N > S, or path nodes not
 *   strictly increasing within [1, N-1] is left untouched and gets
 *   new_len[b] = -1 (this includes d = -2, a verify that timed out).
 *   Limits: 1 <= N <= 64, N <= S, N * D * elem_bytes <= 32768. */
int spec_kv_commit(void *kv, void *mirror, int elem_bytes, int L, int B, int H, int S, int D,
                   const int32_t *cache_len, const int32_t *path_len,
                   const int32_t *path_nodes, int N, int32_t *new_len, hipStream_t stream);

/* Static description of a status code (host). */
const char *spec_status_string(int status);

/* Profiling hook (host, not thread-safe): between begin and end, every call
 * records a HIP event pair around its logit-streaming kernel on the call's
 * stream.  end() waits for those events and returns the summed kernel time
 * in milliseconds and the number of launches timed.  At most `max_launches`
 * launches are timed.  Returns SPEC_OK or SPEC_ERR_HIP / SPEC_ERR_PARAM. */
int spec_profile_begin(int max_launches);
int spec_profile_end(double *total_ms, int *launches);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
