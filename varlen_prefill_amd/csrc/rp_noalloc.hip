// rp_run_noalloc: rp_run with the split-KV workspace in a fixed device array
// of the library, for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array `scratch` is a file-scope __device__ object: every device the
// library runs on holds its own copy (kNoAllocScratchBytes) from module load
// until the process ends.  In host code its name is only a stand-in for the
// symbol, never a device address; the address of a device's copy is looked
// up once per device with hipGetSymbolAddress (that device current) and kept
// in scratch_ptr, which is what the kernels receive.
//
// Partial states are always written by the tile kernel before the merge
// kernel reads them, so nothing in the array needs clearing.  Calls on one
// device share its array: calls that overlap in time (other streams, other
// host threads) race on it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "ragged_prefill.h"
#include "rp_api_internal.h"

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;  // 32 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
void *scratch_ptr[kMaxDevices];  // per device; null until looked up

}  // namespace

extern "C" int rp_run_noalloc(const rp_plan *plan, const void *q, const void *k, const void *v,
                              void *o, float *lse, float sm_scale, void *stream)
{
    if (plan == nullptr)
        return rp::record_error(RP_EINVAL, "plan must not be NULL");
    const size_t need = rp_plan_workspace_bytes(plan);
    if (need > kNoAllocScratchBytes) {
        char msg[200];
        std::snprintf(msg, sizeof msg,
                      "plan needs %zu bytes of split-KV workspace; rp_run_noalloc holds at most "
                      "%zu bytes per device (use rp_run with a workspace)",
                      need, kNoAllocScratchBytes);
        return rp::record_error(RP_EUNSUPPORTED, msg);
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return rp::record_error(RP_EDEVICE, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return rp::record_error(RP_EUNSUPPORTED, "device index beyond 63");
    void *ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        if (scratch_ptr[dev] == nullptr) {
            void *ptr = nullptr;
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || ptr == nullptr)
                return rp::record_error(RP_EDEVICE, e != hipSuccess ? hipGetErrorString(e)
                                                                    : "scratch symbol has no address");
            scratch_ptr[dev] = ptr;
        }
        ws = scratch_ptr[dev];
    }
    return rp::run_plan_on(plan, q, k, v, o, lse, sm_scale, ws, kNoAllocScratchBytes, stream);
}
