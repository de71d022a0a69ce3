// Host-side launchers of the SparsePR kernels (internal; enqueue only, no synchronisation).
#pragma once
#include <hip/hip_runtime.h>
#include "plan_state.h"

namespace spr {

void launch_plan(const void* q, const void* k, const Dims& D, const Bufs& B, hipStream_t s);
void launch_plan_warm(const void* q, const void* k, const Dims& D, const Bufs& B, hipStream_t s);
void launch_plan_from_labels(const void* q, const void* k, const int* klab, const int* qlab,
                             const long long* mass, const Dims& D, const Bufs& B, hipStream_t s);
void launch_route_probes(const Dims& D, const Bufs& B, hipStream_t s);
void launch_identity_plan(const Dims& D, const Bufs& B, hipStream_t s);
void launch_pair_tiles(const Dims& D, const Bufs& B, hipStream_t s);
void launch_set_probes(const Dims& D, const Bufs& B, const int* probes, const float* weights, hipStream_t s);
void launch_permute_kv(const void* k, const void* v, const Dims& D, const Bufs& B, const int* perm, hipStream_t s);
void launch_attend_sparse(const void* q, const Dims& D, const Bufs& B, void* o_sparse, float* o_probe_sparse,
                          hipStream_t s, bool dense = false);
void launch_attend_probes(const void* q, const Dims& D, const Bufs& B, float* o_probe_dense, hipStream_t s);
void launch_residual_projector(const Dims& D, const Bufs& B, hipStream_t s);
void launch_fit(const Dims& D, const Bufs& B, const float* o_psp, const float* o_dn, const float* w, float* coeffs,
                hipStream_t s);
void launch_apply(const Dims& D, const Bufs& B, const void* o_sp, const float* o_dn, const float* coeffs, void* out,
                  hipStream_t s);

}  // namespace spr
