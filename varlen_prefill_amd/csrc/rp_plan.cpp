// Host planner: turns ragged offsets into a balanced tile worklist.
//
// Tiles: each request's query tokens are cut into tiles of kTileRows / g
// tokens (g = GQA group size), one tile per (token range, kv head).  KV is cut
// into canonical chunks of kv_chunk keys at request-relative offsets.  A tile
// whose visible keys reach past one chunk is either split (one work item per
// chunk, each writing an fp32 partial state, and one merge item: split-KV,
// page "vllm-rlt PR #112", results notes: split-KV parallelism pays off for
// few requests) or folded (one work item that runs the chunks in order and
// folds their states itself).  Both give the same bits; the split mode (or,
// in the automatic mode, whether the grid fills the GPU without splitting)
// picks the placement.
// Items are ordered longest-first (LPT), so the hardware's in-order workgroup
// dispatch approximates greedy longest-processing-time scheduling.
//
// Decode-like requests (at most kDecodeRows query rows: qo_len x group) use
// chunks of min(kv_chunk, kDecodeChunk) keys: one tile per kv head would scan
// all of their keys serially (the split-KV of decode at low concurrency, page
// "vllm-rlt PR #112", results notes).
//
// The chunk grid is a property of the request alone (its own qo_len and the
// batch-wide head shape), which keeps per-request results independent of the
// batch ("balanced tile worklist" with automatic split-KV, page
// "flashinfer-ai/flashinfer", attention API, task-scheduled attention).
#include "rp_plan.h"

#include <algorithm>
#include <map>
#include <numeric>
#include <tuple>

namespace rp {

namespace {

constexpr int kOk = 0;
constexpr int kEInval = -1;
constexpr int kEUnsupported = -2;

int64_t limit_of(int64_t i, int64_t qo_len, int64_t kv_len, bool causal)
{
    if (!causal)
        return kv_len;
    int64_t lim = i + kv_len - qo_len + 1;
    return lim < 0 ? 0 : (lim > kv_len ? kv_len : lim);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Launch order.  Workgroups are handed to the XCDs round-robin (workgroup b
// runs on XCD b % X), each XCD with its own L2.  Tiles that read the same K/V
// (same request, kv head and KV chunk) are placed on one XCD when its load
// allows, so their K/V blocks are L2 hits; each XCD's list is longest-first
// (LPT) and the XCD loads are balanced greedily.  Lists are interleaved into
// one grid, padded with empty items (n_tok = 0) to equal length.
void order_items(std::vector<Item> &items, int xcds)
{
    std::stable_sort(items.begin(), items.end(),
                     [](const Item &x, const Item &y) { return x.cost > y.cost; });
    if (xcds <= 1 || items.size() < 2)
        return;
    int64_t total = 0;
    for (const Item &it : items)
        total += it.cost;
    const int64_t target = (total + xcds - 1) / xcds;
    std::vector<int64_t> load((size_t)xcds, 0);
    std::vector<std::vector<Item>> lists((size_t)xcds);
    std::map<std::tuple<int, int, int, int>, int> home;  // (request, kv head, chunk, split) -> XCD
    for (const Item &it : items) {
        const bool partial = it.slot >= 0 && it.fold_keys == 0;
        const auto key = std::make_tuple(it.request, it.kv_head, partial ? it.chunk : 0, partial ? 1 : 0);
        auto h = home.find(key);
        int x;
        if (h != home.end() && load[(size_t)h->second] + it.cost <= target) {
            x = h->second;
        } else {
            x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
            if (h == home.end())
                home.emplace(key, x);
        }
        lists[(size_t)x].push_back(it);
        load[(size_t)x] += it.cost;
    }
    size_t len = 0;
    for (const auto &l : lists)
        len = std::max(len, l.size());
    Item empty{};
    empty.n_tok = 0;
    empty.key_begin = 0;
    empty.key_end = 0;
    empty.slot = -1;
    empty.request = -1;
    items.clear();
    items.reserve(len * (size_t)xcds);
    for (size_t k = 0; k < len; ++k)
        for (int x = 0; x < xcds; ++x)
            items.push_back(k < lists[(size_t)x].size() ? lists[(size_t)x][k] : empty);
}

}  // namespace

int64_t visible_keys(int64_t i, int64_t qo_len, int64_t kv_len, bool causal)
{
    return limit_of(i, qo_len, kv_len, causal);
}

size_t HostPlan::part_o_bytes() const
{
    return (size_t)num_slots * kTileRows * (size_t)shape.head_dim * sizeof(float);
}

size_t HostPlan::workspace_bytes() const
{
    if (num_slots == 0)
        return 0;
    return align256(part_o_bytes()) + align256((size_t)num_slots * kTileRows * sizeof(float));
}

int build_plan(const int32_t *q_indptr, const int32_t *kv_indptr, const PlanShape &shape_in,
               HostPlan &out, std::string &err)
{
    PlanShape shape = shape_in;
    if (shape.kv_chunk == 0)
        shape.kv_chunk = kDefaultKvChunk;
    if (shape.batch < 0) {
        err = "batch must be >= 0";
        return kEInval;
    }
    if (shape.num_qo_heads <= 0 || shape.num_kv_heads <= 0) {
        err = "head counts must be positive";
        return kEInval;
    }
    if (shape.num_qo_heads % shape.num_kv_heads != 0) {
        err = "num_qo_heads must be a multiple of num_kv_heads";
        return kEInval;
    }
    const int group = shape.num_qo_heads / shape.num_kv_heads;
    if (group > kTileRows) {
        err = "GQA group size (num_qo_heads / num_kv_heads) above 128 is not supported";
        return kEUnsupported;
    }
    if (shape.head_dim != 128 && shape.head_dim != 256) {
        err = "head_dim must be 128 or 256";
        return kEUnsupported;
    }
    if (shape.causal != 0 && shape.causal != 1) {
        err = "causal must be 0 or 1";
        return kEInval;
    }
    if (shape.kv_chunk < kChunkAlign || shape.kv_chunk % kChunkAlign != 0) {
        err = "kv_chunk must be a positive multiple of 64";
        return kEInval;
    }
    // Default launch order: XCD-grouped at both head dims (at head_dim 256
    // the 16-row-wave kernel measured 1.7 % faster grouped on the causal
    // workload, neutral non-causal; num_xcds = 1 gives plain longest-first).
    if (shape.num_xcds == 0)
        shape.num_xcds = kDefaultXcds;
    if (shape.num_xcds < 1 || shape.num_xcds > 64) {
        err = "num_xcds must be in [1, 64] (0 = default)";
        return kEInval;
    }
    if (shape.split_mode < 0 || shape.split_mode > 2) {
        err = "unknown split_mode (0 = auto, 1 = never, 2 = always)";
        return kEInval;
    }
    if (shape.batch > 0 && (q_indptr == nullptr || kv_indptr == nullptr)) {
        err = "q_indptr and kv_indptr must not be NULL when batch > 0";
        return kEInval;
    }
    if (shape.batch > 0 && (q_indptr[0] < 0 || kv_indptr[0] < 0)) {
        err = "indptr entries must be >= 0";
        return kEInval;
    }
    for (int b = 0; b < shape.batch; ++b) {
        if (q_indptr[b + 1] < q_indptr[b] || kv_indptr[b + 1] < kv_indptr[b]) {
            err = "indptr must be non-decreasing (request " + std::to_string(b) + ")";
            return kEInval;
        }
    }

    HostPlan plan;
    plan.shape = shape;
    plan.tile_tokens = kTileRows / group;
    const int bk = key_block(shape.head_dim);
    const bool causal = shape.causal != 0;
    const int64_t C_prefill = shape.kv_chunk;
    const int64_t C_decode = std::min<int64_t>(shape.kv_chunk, kDecodeChunk);

    if (shape.batch > 0) {
        plan.max_q_row = q_indptr[shape.batch];
        plan.max_kv_row = kv_indptr[shape.batch];
        plan.total_q = (int64_t)q_indptr[shape.batch] - q_indptr[0];
        plan.total_kv = (int64_t)kv_indptr[shape.batch] - kv_indptr[0];
    }

    // cost of a work item over keys [k0, k1): two MFMA halves per key block,
    // one more where the kernel is expected to split P (tiles whose rows see
    // few keys), plus a fixed epilogue share
    auto item_cost = [&](int64_t k0, int64_t k1, int64_t lim_first) {
        int64_t cost = 4;
        if (k1 > k0)
            cost += ((k1 + bk - 1) / bk - k0 / bk) * (lim_first <= kHiLoKeys ? 3 : 2);
        return cost;
    };
    // tiles in batch order: (tile item over all its keys, chunk size, chunk
    // count); multi-chunk tiles are split or folded below
    struct TileKeys {
        Item it;
        int64_t C;
        int64_t n_chunks;
    };
    std::vector<TileKeys> tiles;
    int64_t total_cost = 0, max_fold_cost = 0;

    double pairs_total = 0.0;
    for (int b = 0; b < shape.batch; ++b) {
        const int64_t qo = (int64_t)q_indptr[b + 1] - q_indptr[b];
        const int64_t kv = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
        for (int64_t i = 0; i < qo; ++i)
            pairs_total += (double)limit_of(i, qo, kv, causal);
        if (qo == 0)
            continue;
        const int64_t C = qo * group <= kDecodeRows ? C_decode : C_prefill;
        for (int64_t t0 = 0; t0 < qo; t0 += plan.tile_tokens) {
            const int64_t n_tok = std::min<int64_t>(plan.tile_tokens, qo - t0);
            const int64_t lim_first = limit_of(t0, qo, kv, causal);
            const int64_t lim_last = limit_of(t0 + n_tok - 1, qo, kv, causal);
            const int64_t key_end = lim_last;
            const int64_t n_chunks = key_end > 0 ? (key_end + C - 1) / C : 0;
            int64_t cost = 0;   // summed over the chunks (the folded item's cost)
            for (int64_t ch = 0; ch < std::max<int64_t>(n_chunks, 1); ++ch)
                cost += item_cost(ch * C, std::min<int64_t>((ch + 1) * C, key_end), lim_first);
            for (int kvh = 0; kvh < shape.num_kv_heads; ++kvh) {
                Item it{};
                it.q_tok0 = (int32_t)(q_indptr[b] + t0);
                it.n_tok = (int32_t)n_tok;
                it.t0 = (int32_t)t0;
                it.qo_len = (int32_t)qo;
                it.kv_row0 = kv_indptr[b];
                it.kv_len = (int32_t)kv;
                it.kv_head = kvh;
                it.request = b;
                it.lim_first = (int32_t)lim_first;
                it.key_begin = 0;
                it.key_end = (int32_t)key_end;
                it.chunk = (int32_t)n_chunks;
                it.slot = -1;
                tiles.push_back({it, C, n_chunks});
                total_cost += cost;
                if (n_chunks > 1)
                    max_fold_cost = std::max(max_fold_cost, cost);
            }
        }
    }

    // placement of the multi-chunk tiles: RP_SPLIT_NEVER folds, RP_SPLIT_ALWAYS
    // splits, the automatic mode folds at head_dim 128 when the grid fills the
    // GPU without split-KV
    bool fold = shape.split_mode == 1;
    if (shape.split_mode == 0)
        fold = shape.head_dim == 128 && max_fold_cost * kResidentTiles128 <= total_cost;
    for (const TileKeys &tk : tiles) {
        const Item &it = tk.it;
        if (tk.n_chunks <= 1) {
            plan.items.push_back(it);
        } else if (fold) {
            Item fi = it;
            fi.slot = (int32_t)plan.num_slots;
            fi.fold_keys = (int32_t)tk.C;
            plan.num_slots += 1;
            plan.items.push_back(fi);
            ++plan.num_fold_items;
        } else {
            const int64_t slot0 = plan.num_slots;
            plan.num_slots += tk.n_chunks;
            for (int64_t ch = 0; ch < tk.n_chunks; ++ch) {
                Item pi = it;
                pi.key_begin = (int32_t)(ch * tk.C);
                pi.key_end = (int32_t)std::min<int64_t>((ch + 1) * tk.C, it.key_end);
                pi.slot = (int32_t)(slot0 + ch);
                pi.chunk = (int32_t)ch;
                plan.items.push_back(pi);
                ++plan.num_partial_items;
            }
            MergeItem mi{};
            mi.q_tok0 = it.q_tok0;
            mi.n_tok = it.n_tok;
            mi.kv_head = it.kv_head;
            mi.slot0 = (int32_t)slot0;
            mi.n_chunks = (int32_t)tk.n_chunks;
            mi.request = it.request;
            plan.merges.push_back(mi);
        }
    }
    if (plan.num_slots > (int64_t)INT32_MAX / kTileRows) {
        err = "too many partial states";
        return kEUnsupported;
    }

    for (Item &it : plan.items) {
        int64_t cost = 0;
        if (it.fold_keys > 0) {
            for (int64_t k0 = it.key_begin; k0 < it.key_end; k0 += it.fold_keys)
                cost += item_cost(k0, std::min<int64_t>(k0 + it.fold_keys, it.key_end), it.lim_first);
        } else {
            cost = item_cost(it.key_begin, it.key_end, it.lim_first);
        }
        it.cost = (int32_t)std::min<int64_t>(cost, INT32_MAX);
    }
    order_items(plan.items, shape.num_xcds);

    const double hd = shape.head_dim;
    plan.flops = 4.0 * hd * shape.num_qo_heads * pairs_total;
    plan.bytes = 2.0 * hd * (2.0 * shape.num_qo_heads * (double)plan.total_q +
                             2.0 * shape.num_kv_heads * (double)plan.total_kv) +
                 4.0 * shape.num_qo_heads * (double)plan.total_q;
    out = std::move(plan);
    return kOk;
}

}  // namespace rp
