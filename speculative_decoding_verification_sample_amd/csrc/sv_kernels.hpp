// Host-side launchers of the verify kernels (internal to libspecverify.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_layout.hpp"

namespace sv {

// logit streaming (sv_stream.hip)
hipError_t launch_softmax_partial(const void *target, const void *draft, int dtype,
                                  int rows_t, int rows_d, int V, int S, Scale k,
                                  float *part_m, double *part_z, hipStream_t stream);
hipError_t launch_argmax_partial(const void *logits, int dtype, int rows, int V, int S,
                                 uint64_t *part_key, hipStream_t stream);

// top-p nucleus threshold per row (sv_topp.hip)
hipError_t launch_topp_select(const void *target, const void *draft, int dtype, int rows_t,
                              int rows_d, int V, int S, Scale k, double k64, double top_p,
                              const float *part_m, const double *part_z, RowStat *rowstat,
                              hipStream_t stream);

// sampling decide / residual / inverse CDF (sv_sample.hip)
hipError_t launch_sample_decide(const void *target, const void *draft, int dtype,
                                const int32_t *tokens, const float *u_accept, int B, int K,
                                int V, int S, double k64, const float *part_m,
                                const double *part_z, const RowStat *rowstat,
                                int32_t *out_accepted, int32_t *out_tokens, float *out_p,
                                float *out_q, Decision *dec, hipStream_t stream);
hipError_t launch_resid_partial(const void *target, const void *draft, int dtype, int B,
                                int K, int V, int S, Scale k, const Decision *dec,
                                ResidPart *rpart, hipStream_t stream);
hipError_t launch_sample_locate(const void *target, const void *draft, int dtype,
                                const float *u_sample, int B, int K, int V, int S, Scale k,
                                const Decision *dec, const ResidPart *rpart,
                                int32_t *out_tokens, float *out_mass, hipStream_t stream);

// greedy and tree decisions (sv_greedy.hip)
hipError_t launch_greedy_decide(const int32_t *tokens, int B, int K, int S,
                                const uint64_t *part_key, int32_t *out_accepted,
                                int32_t *out_tokens, hipStream_t stream);
hipError_t launch_tree_decide(const int32_t *parents, const int32_t *node_tokens,
                              const uint8_t *anc_mask, int B, int N, int S,
                              const uint64_t *part_key, int32_t *out_path_len,
                              int32_t *out_path_nodes, int32_t *out_tokens,
                              hipStream_t stream);

}  // namespace sv
