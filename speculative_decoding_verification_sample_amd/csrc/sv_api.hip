// extern "C" entry points of libspecverify.so (declared in include/spec_verify.h).
// Every argument is validated on the host before the first HIP call, so an
// invalid call returns an error code with nothing enqueued.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "spec_verify.h"
#include "sv_kernels.hpp"
#include "sv_layout.hpp"

namespace {

using sv::Layout;
using sv::Scale;

constexpr int kMaxK = 63;
constexpr int kMaxN = 64;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(long B, long KN, long V, int op) {
  if (B < 1 || V < 1 || V > 0x7FFFFFFFL) return SPEC_ERR_SHAPE;
  if (op == SPEC_OP_TREE) {
    if (KN < 1 || KN > kMaxN) return SPEC_ERR_SHAPE;
  } else if (KN < 1 || KN > kMaxK) {
    return SPEC_ERR_SHAPE;
  }
  // one workgroup per (row, split) on a 1-D grid
  const long rows = op == SPEC_OP_SAMPLE ? B * (2 * KN + 1) : op == SPEC_OP_GREEDY ? B * (KN + 1) : B * KN;
  if (B > 0x7FFFFFFFL || rows > 0x7FFFFFFFL) return SPEC_ERR_SHAPE;
  const long S = sv::num_splits((int)V, SPEC_F32);  // the f32 split count is the larger one
  if (rows * S > 0x7FFFFFFFL) return SPEC_ERR_SHAPE;
  if (op == SPEC_OP_SAMPLE && B * (long)sv::num_splits_b((int)V, SPEC_F32) + rows * S > 0x7FFFFFFFL)
    return SPEC_ERR_SHAPE;
  // the draw stages a request's residual splits in LDS
  if (op == SPEC_OP_SAMPLE && sv::num_splits_b((int)V, SPEC_F32) > sv::kMaxSplitsB)
    return SPEC_ERR_SHAPE;
  return SPEC_OK;
}

// Every call tags its partials with a fresh 64-bit epoch.  The sequence
// starts from a scrambled clock reading so that tags left in reused memory by
// another process do not match.
std::atomic<uint64_t> g_epoch{(uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() *
                              0x9E3779B97F4A7C15ull};

sv::u64 next_epoch() {
  sv::u64 e = g_epoch.fetch_add(0x9E3779B97F4A7C15ull);
  return e ? e : 1;
}

bool dtype_ok(int dtype) { return dtype == SPEC_F32 || dtype == SPEC_BF16; }

int check_workspace(void *ws, size_t bytes, const Layout &L) {
  if (L.total > 0 && !ws) return SPEC_ERR_NULL;
  if (!aligned(ws, 256)) return SPEC_ERR_ALIGN;
  if (bytes < L.total) return SPEC_ERR_WORKSPACE;
  return SPEC_OK;
}

template <class T>
T *carve(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

// ---- profiling hook: events around the logit-streaming kernel ----
struct Profile {
  bool active = false;
  int max = 0;
  std::vector<hipEvent_t> ev;  // pairs
  int used = 0;
} g_prof;

void prof_before(hipStream_t s) {
  if (g_prof.active && g_prof.used < g_prof.max) (void)hipEventRecord(g_prof.ev[2 * g_prof.used], s);
}
void prof_after(hipStream_t s) {
  if (g_prof.active && g_prof.used < g_prof.max) {
    (void)hipEventRecord(g_prof.ev[2 * g_prof.used + 1], s);
    ++g_prof.used;
  }
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_bytes(int op, int B, int K_or_N, int V, int dtype, int use_top_p) {
  if (op != SPEC_OP_GREEDY && op != SPEC_OP_SAMPLE && op != SPEC_OP_TREE) return 0;
  if (!dtype_ok(dtype) || check_shape(B, K_or_N, V, op) != SPEC_OK) return 0;
  return sv::make_layout(op, B, K_or_N, V, dtype, use_top_p ? 1 : 0).total;
}

const char *spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_NULL: return "a required pointer is NULL";
    case SPEC_ERR_SHAPE: return "B, K, N or V out of range";
    case SPEC_ERR_PARAM: return "bad temperature, top_p, dtype or op";
    case SPEC_ERR_WORKSPACE: return "workspace too small";
    case SPEC_ERR_ALIGN: return "misaligned workspace or logits";
    case SPEC_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int spec_verify_greedy(const void *target_logits, int dtype, const int32_t *draft_tokens, int B,
                       int K, int V, int32_t *out_accepted, int32_t *out_tokens, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (!target_logits || !draft_tokens || !out_accepted || !out_tokens) return SPEC_ERR_NULL;
  if (!dtype_ok(dtype)) return SPEC_ERR_PARAM;
  int rc = check_shape(B, K, V, SPEC_OP_GREEDY);
  if (rc) return rc;
  if (!aligned(target_logits, sv::elem_bytes(dtype))) return SPEC_ERR_ALIGN;
  const Layout L = sv::make_layout(SPEC_OP_GREEDY, B, K, V, dtype, 0);
  if ((rc = check_workspace(workspace, workspace_bytes, L))) return rc;
  uint64_t *part_key = carve<uint64_t>(workspace, L.part_key);
  sv::u64 *part_tag = carve<sv::u64>(workspace, L.part_tag);
  prof_before(stream);
  if (sv::launch_greedy(target_logits, dtype, draft_tokens, B, K, V, L.S, next_epoch(), part_key,
                        part_tag, out_accepted, out_tokens, stream) != hipSuccess)
    return SPEC_ERR_HIP;
  prof_after(stream);
  return SPEC_OK;
}

}  // extern "C"

namespace {

// The sampling call with batch-wide (temps == NULL) or per-request
// parameters; arguments already validated except the workspace.
int run_sample(const void *target_logits, const void *draft_logits, int dtype,
               const int32_t *draft_tokens, const float *u_accept, const float *u_sample,
               double k64, float top_p, const float *temps, const float *topps, int B, int K,
               int V, int32_t *out_accepted, int32_t *out_tokens, float *out_p_draft,
               float *out_q_draft, float *out_residual_mass, void *workspace,
               size_t workspace_bytes, hipStream_t stream) {
  const bool use_top_p = topps != nullptr || top_p < 1.0f;
  const Layout L = sv::make_layout(SPEC_OP_SAMPLE, B, K, V, dtype, use_top_p);
  int rc;
  if ((rc = check_workspace(workspace, workspace_bytes, L))) return rc;
  sv::SampleArgs a;
  a.target = (const char *)target_logits;
  a.draft = (const char *)draft_logits;
  a.tokens = draft_tokens;
  a.u_accept = u_accept;
  a.u_sample = u_sample;
  a.temps = temps;
  a.topps = topps;
  a.B = B;
  a.K = K;
  a.V = V;
  a.S = L.S;
  a.SB = L.SB;
  a.k64 = k64;
  a.top_p = (double)top_p;
  a.k = sv::make_scale(k64);
  a.epoch = next_epoch();
  a.part_m = carve<sv::u64>(workspace, L.part_m);
  a.part_z = carve<sv::u64>(workspace, L.part_z);
  a.part_x = carve<sv::u64>(workspace, L.part_x);
  a.rowstat = use_top_p ? carve<sv::RowStat>(workspace, L.rowstat) : nullptr;
  a.rtot = carve<sv::u64>(workspace, L.rtot);
  a.part_h = use_top_p ? carve<uint8_t>(workspace, L.part_h) : nullptr;
  a.part_c = use_top_p ? carve<uint32_t>(workspace, L.part_c) : nullptr;
  a.part_c2 = use_top_p ? carve<uint16_t>(workspace, L.part_c2) : nullptr;
  a.topband = use_top_p ? carve<sv::TopBand>(workspace, L.topband) : nullptr;
  a.band_n = use_top_p ? carve<unsigned>(workspace, L.band_n) : nullptr;
  a.band_keys = use_top_p ? carve<uint32_t>(workspace, L.band_keys) : nullptr;
  a.band_above = use_top_p ? carve<double>(workspace, L.band_above) : nullptr;
  // top-p with batch-wide parameters: the ratio tests once per request, in
  // their own launch before the residual tiles
  a.dec = use_top_p && temps == nullptr ? carve<sv::Decision>(workspace, L.dec) : nullptr;
  a.out_accepted = out_accepted;
  a.out_tokens = out_tokens;
  a.out_p = out_p_draft;
  a.out_q = out_q_draft;
  a.out_mass = out_residual_mass;
  // residual tiles trail their request's streaming tiles by about one
  // resident wave of requests
  a.lag = sv::resident_workgroups(dtype) / ((2 * K + 1) * L.S) + 1;
  a.phase = use_top_p ? 1 : 0;
  prof_before(stream);
  if (sv::launch_sample(a, dtype, stream) != hipSuccess) return SPEC_ERR_HIP;
  prof_after(stream);
  if (use_top_p) {
    if (sv::launch_topp_select(a, dtype, stream) != hipSuccess) return SPEC_ERR_HIP;
    if (a.dec) {  // batch-wide parameters: decide, residual masses, draw
      if (sv::launch_topp_decide(a, stream) != hipSuccess ||
          sv::launch_topp_residual(a, dtype, stream) != hipSuccess)
        return SPEC_ERR_HIP;
      return SPEC_OK;
    }
    a.phase = 2;
    if (sv::launch_sample(a, dtype, stream) != hipSuccess) return SPEC_ERR_HIP;
  }
  return SPEC_OK;
}

int check_sample_args(const void *target_logits, const void *draft_logits, int dtype,
                      const int32_t *draft_tokens, const float *u_accept, const float *u_sample,
                      int B, int K, int V, int32_t *out_accepted, int32_t *out_tokens) {
  if (!target_logits || !draft_logits || !draft_tokens || !u_accept || !u_sample ||
      !out_accepted || !out_tokens)
    return SPEC_ERR_NULL;
  if (!dtype_ok(dtype)) return SPEC_ERR_PARAM;
  int rc = check_shape(B, K, V, SPEC_OP_SAMPLE);
  if (rc) return rc;
  if (!aligned(target_logits, sv::elem_bytes(dtype)) || !aligned(draft_logits, sv::elem_bytes(dtype)))
    return SPEC_ERR_ALIGN;
  return SPEC_OK;
}

}  // namespace

extern "C" {

int spec_verify_sample(const void *target_logits, const void *draft_logits, int dtype,
                       const int32_t *draft_tokens, const float *u_accept,
                       const float *u_sample, float temperature, float top_p, int B, int K,
                       int V, int32_t *out_accepted, int32_t *out_tokens, float *out_p_draft,
                       float *out_q_draft, float *out_residual_mass, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  int rc = check_sample_args(target_logits, draft_logits, dtype, draft_tokens, u_accept,
                             u_sample, B, K, V, out_accepted, out_tokens);
  if (rc) return rc;
  if (!std::isfinite(temperature) || !(temperature > 0.0f)) return SPEC_ERR_PARAM;
  if (!(top_p > 0.0f) || !(top_p <= 1.0f)) return SPEC_ERR_PARAM;
  const double k64 = sv::kLog2e / (double)temperature;  // log2(e) / T
  if (!std::isfinite(k64) || !(k64 > 0.0) || k64 > 3.0e38) return SPEC_ERR_PARAM;
  return run_sample(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample, k64,
                    top_p, nullptr, nullptr, B, K, V, out_accepted, out_tokens, out_p_draft,
                    out_q_draft, out_residual_mass, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- the sampling call on a library-held workspace ----
// One array per GPU, in device memory, for callers that cannot allocate.
// In host code `scratch` names a host-side stand-in, not a device address:
// the device address comes from hipGetSymbolAddress, once per device, with
// that device current, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[SPEC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch` (its device address); looked up on
// the first call on that device.
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPEC_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPEC_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SPEC_OK;
}

}  // namespace

extern "C" {

int spec_verify_sample_noalloc(const void *target_logits, const void *draft_logits, int dtype,
                               const int32_t *draft_tokens, const float *u_accept,
                               const float *u_sample, float temperature, float top_p, int B,
                               int K, int V, int32_t *out_accepted, int32_t *out_tokens,
                               float *out_p_draft, float *out_q_draft,
                               float *out_residual_mass, hipStream_t stream) {
  int rc = check_sample_args(target_logits, draft_logits, dtype, draft_tokens, u_accept,
                             u_sample, B, K, V, out_accepted, out_tokens);
  if (rc) return rc;
  if (!std::isfinite(temperature) || !(temperature > 0.0f)) return SPEC_ERR_PARAM;
  if (!(top_p > 0.0f) || !(top_p <= 1.0f)) return SPEC_ERR_PARAM;
  const double k64 = sv::kLog2e / (double)temperature;
  if (!std::isfinite(k64) || !(k64 > 0.0) || k64 > 3.0e38) return SPEC_ERR_PARAM;
  const Layout L = sv::make_layout(SPEC_OP_SAMPLE, B, K, V, dtype, top_p < 1.0f);
  if (L.total > (size_t)SPEC_SCRATCH_BYTES) return SPEC_ERR_WORKSPACE;
  void *ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return run_sample(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample, k64,
                    top_p, nullptr, nullptr, B, K, V, out_accepted, out_tokens, out_p_draft,
                    out_q_draft, out_residual_mass, ws, (size_t)SPEC_SCRATCH_BYTES, stream);
}

int spec_verify_mixed(const void *target_logits, const void *draft_logits, int dtype,
                      const int32_t *draft_tokens, const float *u_accept, const float *u_sample,
                      const float *temperature, const float *top_p, int B, int K, int V,
                      int32_t *out_accepted, int32_t *out_tokens, float *out_p_draft,
                      float *out_q_draft, float *out_residual_mass, void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  int rc = check_sample_args(target_logits, draft_logits, dtype, draft_tokens, u_accept,
                             u_sample, B, K, V, out_accepted, out_tokens);
  if (rc) return rc;
  if (!temperature) return SPEC_ERR_NULL;
  return run_sample(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample, 1.0,
                    1.0f, temperature, top_p, B, K, V, out_accepted, out_tokens, out_p_draft,
                    out_q_draft, out_residual_mass, workspace, workspace_bytes, stream);
}

int spec_verify_tree(const void *target_logits, int dtype, const int32_t *parents,
                     const int32_t *node_tokens, const uint8_t *anc_mask, int B, int N, int V,
                     int32_t *out_path_len, int32_t *out_path_nodes, int32_t *out_tokens,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!target_logits || !parents || !node_tokens || !anc_mask || !out_path_len ||
      !out_path_nodes || !out_tokens)
    return SPEC_ERR_NULL;
  if (!dtype_ok(dtype)) return SPEC_ERR_PARAM;
  int rc = check_shape(B, N, V, SPEC_OP_TREE);
  if (rc) return rc;
  if (!aligned(target_logits, sv::elem_bytes(dtype))) return SPEC_ERR_ALIGN;
  const Layout L = sv::make_layout(SPEC_OP_TREE, B, N, V, dtype, 0);
  if ((rc = check_workspace(workspace, workspace_bytes, L))) return rc;
  uint64_t *part_key = carve<uint64_t>(workspace, L.part_key);
  sv::u64 *part_tag = carve<sv::u64>(workspace, L.part_tag);
  prof_before(stream);
  if (sv::launch_tree(target_logits, dtype, parents, node_tokens, anc_mask, B, N, V, L.S,
                      next_epoch(), part_key, part_tag, out_path_len, out_path_nodes, out_tokens,
                      stream) != hipSuccess)
    return SPEC_ERR_HIP;
  prof_after(stream);
  return SPEC_OK;
}

// ---- LM head fused with greedy verification ----
static int lmhead_shape(long B, long K, long d, long V) {
  if (B < 1 || K < 1 || K > kMaxK || d < 64 || d % 64 != 0 || d > (1L << 20) || V < 1 ||
      V > 0x7FFFFFFFL)
    return SPEC_ERR_SHAPE;
  const long M = B * (K + 1);
  const long RT = (M + 383) / 384, VT = sv::lmhead_vocab_tiles((int)V);
  if (M > (1L << 24) || (VT + 7) / 8 * 8 * RT > 0x7FFFFFFFL) return SPEC_ERR_SHAPE;
  return SPEC_OK;
}

size_t spec_lmhead_workspace_bytes(int B, int K, int d, int V) {
  if (lmhead_shape(B, K, d, V) != SPEC_OK) return 0;
  return (size_t)B * (size_t)(K + 1) * (size_t)sv::lmhead_vocab_tiles(V) * sizeof(uint64_t);
}

int spec_lmhead_greedy(const void *hidden, const void *weight, const int32_t *draft_tokens, int B,
                       int K, int d, int V, int32_t *out_accepted, int32_t *out_tokens,
                       int32_t *out_argmax, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (!hidden || !weight || !draft_tokens || !out_accepted || !out_tokens || !workspace)
    return SPEC_ERR_NULL;
  int rc = lmhead_shape(B, K, d, V);
  if (rc) return rc;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(workspace, 256))
    return SPEC_ERR_ALIGN;
  if (workspace_bytes < spec_lmhead_workspace_bytes(B, K, d, V)) return SPEC_ERR_WORKSPACE;
  prof_before(stream);
  const hipError_t e = sv::launch_lmhead_greedy(hidden, weight, draft_tokens, B, K, d, V,
                                                out_accepted, out_tokens, out_argmax,
                                                (uint64_t *)workspace, stream);
  prof_after(stream);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int spec_tree_merge(const int32_t *parents1, const int32_t *tokens1, const float *conf1, int n1,
                    const int32_t *parents2, const int32_t *tokens2, const float *conf2, int n2,
                    int B, int32_t *out_parents, int32_t *out_tokens, uint8_t *out_mask,
                    float *out_conf, int32_t *out_route, hipStream_t stream) {
  if (!parents1 || !tokens1 || !conf1 || !parents2 || !tokens2 || !conf2 || !out_parents ||
      !out_tokens || !out_mask)
    return SPEC_ERR_NULL;
  if (B < 1 || n1 < 0 || n2 < 0 || n1 + n2 + 1 > kMaxN) return SPEC_ERR_SHAPE;
  if (sv::launch_tree_merge(parents1, tokens1, conf1, n1, parents2, tokens2, conf2, n2, B,
                            out_parents, out_tokens, out_mask, out_conf, out_route,
                            stream) != hipSuccess)
    return SPEC_ERR_HIP;
  return SPEC_OK;
}

int spec_kv_commit(void *kv, void *mirror, int elem_bytes, int L, int B, int H, int S, int D,
                   const int32_t *cache_len, const int32_t *path_len, const int32_t *path_nodes,
                   int N, int32_t *new_len, hipStream_t stream) {
  if (!kv || !cache_len || !path_len || !new_len) return SPEC_ERR_NULL;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return SPEC_ERR_PARAM;
  if (L < 1 || B < 1 || H < 1 || S < 1 || D < 1 || N < 1 || N > kMaxN || N > S)
    return SPEC_ERR_SHAPE;
  const size_t row_bytes = (size_t)D * (size_t)elem_bytes;
  if (row_bytes % 16 != 0) return SPEC_ERR_ALIGN;
  if (!aligned(kv, 16) || (mirror && !aligned(mirror, 16))) return SPEC_ERR_ALIGN;
  if (mirror == kv) return SPEC_ERR_PARAM;
  // one head of a cycle (N rows) must fit a workgroup's registers
  const long per_head = (long)N * (long)(row_bytes / 16);
  if (per_head > sv::kv_items_per_wg()) return SPEC_ERR_SHAPE;
  const long groups = (long)L * 2 * B;
  if (groups > 0x7FFFFFFFL) return SPEC_ERR_SHAPE;
  if (sv::launch_kv_commit(kv, mirror, L, B, H, S, row_bytes, cache_len, path_len,
                           path_nodes, N, new_len, stream) != hipSuccess)
    return SPEC_ERR_HIP;
  return SPEC_OK;
}

int spec_profile_begin(int max_launches) {
  if (max_launches < 1 || max_launches > (1 << 20)) return SPEC_ERR_PARAM;
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
  for (auto &e : g_prof.ev)
    if (hipEventCreate(&e) != hipSuccess) return SPEC_ERR_HIP;
  g_prof.max = max_launches;
  g_prof.used = 0;
  g_prof.active = true;
  return SPEC_OK;
}

int spec_profile_end(double *total_ms, int *launches) {
  if (!total_ms || !launches) return SPEC_ERR_NULL;
  double sum = 0.0;
  int rc = SPEC_OK;
  for (int i = 0; i < g_prof.used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess) {
      rc = SPEC_ERR_HIP;
      break;
    }
    sum += ms;
  }
  *total_ms = sum;
  *launches = g_prof.used;
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.active = false;
  g_prof.used = 0;
  g_prof.max = 0;
  return rc;
}

}  // extern "C"
