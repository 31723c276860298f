// Internal entry points shared by the C ABI's stream calls and the step
// graph: argument checks plus one launch into a Sink.
#pragma once

#include <new>

#include "fsdp_mi355x.h"
#include "kernels.hpp"
#include "plan.hpp"

namespace fsdp {

// Runs the body of a C entry point and turns a C++ exception into a status,
// so that none crosses the C ABI: a failed host allocation (argument lists,
// the per-device table map) gives FSDP_ERR_OUT_OF_MEMORY, anything else
// (a lock that cannot be taken) FSDP_ERR_HIP.
template <typename F>
fsdp_status guarded(F&& body) noexcept {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return FSDP_ERR_OUT_OF_MEMORY;
  } catch (...) {
    return FSDP_ERR_HIP;
  }
}

// FSDP_OK, or the status a failed HIP call maps to (clearing HIP's error).
fsdp_status status_of(hipError_t e);

// FSDP_OK when the AdamW hyper-parameters are usable: finite lr >= 0,
// 0 <= beta < 1, eps > 0, finite weight decay >= 0.
fsdp_status check_hparams(const fsdp_adamw_hparams* hp);

// The float64 scalars of AdamW step `step` (>= 1).
fsdp_status adam_scalars(const fsdp_adamw_hparams* hp, int64_t step, AdamScalars* sc);

// fsdp_gather_unflatten's checks and launch.
fsdp_status gather_impl(const fsdp_plan* plan, const void* shards, int32_t dtype,
                        void* const* full_out, const Sink& sink);

// fsdp_adamw_shard_step's checks and launch, with the scalars given (sc) or
// read from device memory when the kernel runs (scp non-null).
fsdp_status adamw_impl(const fsdp_plan* plan, const AdamScalars& sc, const AdamScalars* scp,
                       const void* const* grads, int32_t grad_dtype, int32_t grads_are_replicas,
                       float* master, float* m, float* v, void* param_out, int32_t param_dtype,
                       const Sink& sink);

// The fused AdamW step of `plan` (R gradient replicas) and the gather of
// `next` (parameter dtype), in one launch when the step is short, else in
// two; fsdp_adamw_step_then_gather's checks.
fsdp_status adamw_gather_impl(const fsdp_plan* plan, const AdamScalars& sc,
                              const AdamScalars* scp, const void* const* grads,
                              int32_t grad_dtype, float* master, float* m, float* v,
                              void* param_out, int32_t param_dtype, const fsdp_plan* next,
                              const void* next_shards, void* const* full_out, const Sink& sink);

}  // namespace fsdp
