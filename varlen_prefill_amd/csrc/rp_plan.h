// Host planner: ragged offsets -> balanced tile worklist.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "rp_internal.h"

namespace rp {

struct PlanShape {
    int batch = 0;
    int num_qo_heads = 0;
    int num_kv_heads = 0;
    int head_dim = 0;
    int causal = 0;
    int kv_chunk = kDefaultKvChunk;
    int split_mode = 0;  // enum rp_split_mode
    int num_xcds = kDefaultXcds;
};

struct HostPlan {
    PlanShape shape;
    std::vector<Item> items;
    std::vector<MergeItem> merges;
    int64_t num_slots = 0;
    int64_t num_partial_items = 0;
    int64_t num_fold_items = 0;  // items that fold their tile's KV chunks in the workgroup
    int64_t total_q = 0;
    int64_t total_kv = 0;
    int64_t max_q_row = 0;   // q_indptr[batch]: rows Q/O must hold
    int64_t max_kv_row = 0;  // kv_indptr[batch]
    int tile_tokens = 0;
    double flops = 0.0;
    double bytes = 0.0;

    size_t part_o_bytes() const;
    size_t workspace_bytes() const;
};

// Returns 0 (RP_OK) or a negative rp_status; on failure `err` says why.
int build_plan(const int32_t *q_indptr, const int32_t *kv_indptr, const PlanShape &shape,
               HostPlan &out, std::string &err);

// Number of (query, key) pairs visible to one query row (bottom-right causal).
int64_t visible_keys(int64_t i, int64_t qo_len, int64_t kv_len, bool causal);

}  // namespace rp
