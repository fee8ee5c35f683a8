// State-merge kernel: the merge_state / merge_state_in_place / merge_states
// operations of the cascade API (page "flashinfer-ai/flashinfer", cascade API,
// Merge Attention States), and the last step of shared-prefix attention.
//
// HBM-bound elementwise work: per (row, head) it reads num_states values of
// head_dim bf16 plus one fp32 LSE each and writes head_dim bf16 plus one fp32.
// Thread g owns the 8 consecutive elements 8 g .. 8 g + 7 of the flattened
// [rows][heads][head_dim] output (one 16-byte load per state), so consecutive
// lanes read and write consecutive 16-byte pieces.  States are taken in
// groups of four whose loads are all issued before any is used, and folded
// with a running maximum, so a thread keeps several loads in flight.
#include <hip/hip_runtime.h>

#include <cmath>

#include "rp_state_merge.h"

namespace rp {
namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 4;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(kThreads) void state_merge_kernel(StateMergeArgs a, int cpr_log2,
                                                               int64_t total)
{
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= total)
        return;
    const int chunk = (int)(g & ((1 << cpr_log2) - 1));
    const int64_t rh = g >> cpr_log2;
    const int64_t row = rh <= 0xffffffffll ? (int64_t)((uint32_t)rh / (uint32_t)a.num_heads)
                                           : rh / a.num_heads;
    const int h = (int)(rh - row * a.num_heads);

    auto state_s = [&](int i) {
        const float *base = (a.s1 != nullptr && i == 1) ? a.s1 : a.s0 + i * a.s_state_stride;
        return base[row * a.s_row_stride + h];
    };
    auto state_v = [&](int i) {
        const __bf16 *base = (a.v1 != nullptr && i == 1)
                                 ? static_cast<const __bf16 *>(a.v1)
                                 : static_cast<const __bf16 *>(a.v0) + i * a.v_state_stride;
        return *reinterpret_cast<const bf16x8 *>(base + row * a.v_row_stride +
                                                 (int64_t)h * a.head_dim + 8 * chunk);
    };

    // running state: max m, sum of exp(s_i - m), sum of exp(s_i - m) v_i
    float m = -INFINITY, sum = 0.0f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < a.num_states; i0 += kGroup) {
        float sv[kGroup];
        bf16x8 xv[kGroup];
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
            if (i0 + j < a.num_states) {
                sv[j] = state_s(i0 + j);
                xv[j] = state_v(i0 + j);
            }
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            if (i0 + j >= a.num_states)
                break;
            const float mn = fmaxf(m, sv[j]);
            if (mn == -INFINITY)
                continue;  // every state so far is empty
            const float c = expf(m - mn);      // 0 while m = -inf, 1 if the max is unchanged
            const float w = expf(sv[j] - mn);
            sum = fmaf(sum, c, w);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[e] = fmaf(w, (float)xv[j][e], acc[e] * c);
            m = mn;
        }
    }
    const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        out[e] = (__bf16)(acc[e] * inv);
    *reinterpret_cast<bf16x8 *>(static_cast<__bf16 *>(a.v_out) + 8 * g) = out;
    if (a.s_out != nullptr && chunk == 0)
        a.s_out[rh] = m == -INFINITY ? -INFINITY : m + logf(sum);
}

}  // namespace

int launch_state_merge(const StateMergeArgs &args, void *stream)
{
    if (args.rows <= 0 || args.num_heads <= 0)
        return (int)hipSuccess;
    const int cpr_log2 = __builtin_ctz((unsigned)(args.head_dim / 8));
    const int64_t total = (args.rows * args.num_heads) << cpr_log2;
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffff)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(state_merge_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), args, cpr_log2, total);
    return (int)hipGetLastError();
}

}  // namespace rp
