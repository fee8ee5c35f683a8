// Merge of attention states (internal interface between the C ABI and the
// state-merge kernel).  An attention state over a key set is the pair
// (v, s): v the softmax-weighted mean of the values over that set, s the
// natural-log log-sum-exp of its scores.  States over disjoint key sets merge
// into the state over their union (page "flashinfer-ai/flashinfer", cascade
// API, Merge Attention States):
//     s = log(sum_i exp(s_i)),   v = sum_i exp(s_i - s) v_i.
#pragma once

#include <cstdint>

namespace rp {

// State i of row r, head h:
//   v: (v1 != null && i == 1 ? v1 : v0 + i * v_state_stride) + r * v_row_stride + h * head_dim
//   s: (s1 != null && i == 1 ? s1 : s0 + i * s_state_stride) + r * s_row_stride + h
// Output row r, head h: v_out + (r * num_heads + h) * head_dim, s_out + r * num_heads + h.
struct StateMergeArgs {
    const void *v0;
    const void *v1;
    const float *s0;
    const float *s1;
    void *v_out;
    float *s_out;  // may be null
    int64_t v_state_stride, v_row_stride;
    int64_t s_state_stride, s_row_stride;
    int64_t rows;
    int32_t num_heads;
    int32_t head_dim;   // 8 * 2^k, 8..512
    int32_t num_states; // >= 1
};

// hipError_t as int.
int launch_state_merge(const StateMergeArgs &args, void *stream);

}  // namespace rp
