// Library-internal entry points of the host API, shared between the C ABI
// source files (not part of the public ABI).
#pragma once

#include <cstddef>

struct rp_plan;

namespace rp {

// Records `msg` as this thread's last error text and returns `status`.
int record_error(int status, const char *msg);

// rp_run with an explicit split-KV workspace (any plan that rp_run accepts).
int run_plan_on(const rp_plan *plan, const void *q, const void *k, const void *v, void *o,
                float *lse, float sm_scale, void *workspace, size_t workspace_bytes,
                void *stream);

}  // namespace rp
