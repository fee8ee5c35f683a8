// Internal definitions shared by the host library and the gfx950 kernels.
//
// A plan is a list of tile work items.  A tile is a block of up to
// kTileRows "rows" of one request and one kv head, where a row is a
// (query token, qo head) pair: the g = num_qo_heads / num_kv_heads qo heads of a
// GQA group that read the same kv head are packed together, token-major, so a
// single K/V block in LDS serves all of them (GQA as on page "Module
// flashinfer", functions: num_qo_heads a multiple of num_kv_heads).
//
// Each item covers a request-relative key range.  KV is cut into canonical
// chunks of kv_chunk keys at request-relative offsets.  A tile whose visible
// keys span several chunks is split: one item per chunk writes an fp32
// partial state (o_c, lse_c) into the workspace and a merge item folds the
// chunks left to right (the merge of attention states of page
// "flashinfer-ai/flashinfer", "Merge Attention States").  Chunk boundaries
// depend only on the request, never on the batch, so per-request results do
// not change with batch composition.
#pragma once

#include <cstdint>

namespace rp {

constexpr int kTileRows = 128;      // rows per tile: 4 waves x 32 rows (head_dim 128), 8 x 16 (256)
constexpr int kMergeThreads = 256;  // threads per merge workgroup
constexpr int kDefaultKvChunk = 8192;
constexpr int kChunkAlign = 64;     // kv_chunk must be a multiple of this
// Requests whose query rows (qo_len x group) fill at most kDecodeRows rows of a
// tile (decode-like) are cut into chunks of min(kv_chunk, kDecodeChunk) keys:
// their work is a long key scan with few rows, which needs the parallelism.
constexpr int kDecodeRows = 32;
constexpr int kDecodeChunk = 2048;
constexpr int kDefaultXcds = 8;     // MI355X: 8 XCDs, workgroups dispatched round-robin
// Workgroups of the head_dim 128 tile kernel resident at once on an MI355X
// (256 CUs x 2).  The automatic split mode folds a tile's KV chunks in one
// workgroup when the longest folded tile costs no more than the work each of
// these would get on average: the grid then fills the GPU without split-KV.
constexpr int kResidentTiles128 = 512;
// P enters the PV product either rounded to bf16 or split into a bf16 hi part
// and a bf16 lo remainder (two MFMAs, accurate to about 2^-17).
//
// Tiles whose first row sees at most kHiLoKeys keys split P on every block:
// their rows see few keys, so single keys carry much of the softmax.
//
// Other tiles of final (unsplit) items round P to bf16; an item whose result
// holds an output element with |O| >= kRecomputeAbsO is computed again with P
// split on every block.  From 2 up, half a bf16 ulp of O (7.8e-3 in [2, 4))
// leaves almost none of the 8e-3 max-abs gate to the rest of the arithmetic;
// below kRecomputeAbsO it leaves at least 4.1e-3, which the 2^-9 relative
// rounding of the softmax weights reaches only where the weighted mean of
// |V| exceeds 2.1 while |O| stays below 1.5 (large values of both signs
// cancelling under a few dominant keys).
//
// Partial states of split-KV tiles cannot be recomputed after the merge, so
// they split P in the key blocks where some row of the wave has a key whose p
// exceeds kHiLoFracPartial of the row's running sum (the block included):
// every key left rounded ends with a weight of at most that fraction.
constexpr int kHiLoKeys = 128;
#ifndef RP_RECOMPUTE_ABS_O
#define RP_RECOMPUTE_ABS_O 1.5f
#endif
constexpr float kRecomputeAbsO = RP_RECOMPUTE_ABS_O;
constexpr float kHiLoFracPartial = 0.125f;

// Key-block shape of the tile kernel: keys per block and LDS pipeline depth
// (stages in flight, K and V of one block per stage).
#ifndef RP_HD128_BK
#define RP_HD128_BK 32
#endif
#ifndef RP_HD128_STAGES
#define RP_HD128_STAGES 2
#endif
#ifndef RP_HD256_BK
#define RP_HD256_BK 32
#endif
#ifndef RP_HD256_STAGES
#define RP_HD256_STAGES 2
#endif
inline constexpr int key_block(int head_dim) { return head_dim == 128 ? RP_HD128_BK : RP_HD256_BK; }
inline constexpr int kv_stages(int head_dim) { return head_dim == 128 ? RP_HD128_STAGES : RP_HD256_STAGES; }

// Work item of the tile kernel: 16 int32 (64 bytes).
struct Item {
    int32_t q_tok0;     // global row (in Q/O) of the tile's first token
    int32_t n_tok;      // tokens in the tile (>= 1; 0 marks an empty padding item)
    int32_t t0;         // request-relative index of the first token
    int32_t qo_len;     // request's query length
    int32_t kv_row0;    // global row (in K/V) of the request's key 0
    int32_t kv_len;     // request's key length
    int32_t kv_head;    // kv head; qo heads kv_head*g .. kv_head*g+g-1
    int32_t key_begin;  // request-relative first key of this item
    int32_t key_end;    // request-relative end key (exclusive); <= key_begin: no keys
    int32_t slot;       // -1: write final O/LSE; >= 0: partial-state slot (a fold item's running state)
    int32_t request;    // request index in the batch
    int32_t chunk;      // canonical chunk index of a partial item; chunk count otherwise
    int32_t cost;       // planner's cost estimate (key blocks, hi/lo weighted)
    int32_t lim_first;  // keys visible to the tile's first row (causal limit)
    int32_t fold_keys;  // > 0: the workgroup folds the tile's KV chunks of this many keys
                        // itself (running state in slot `slot`, final O/LSE written)
    int32_t reserved1;
};
static_assert(sizeof(Item) == 64, "Item must stay 16 int32");

// Work item of the merge kernel: 8 int32.
struct MergeItem {
    int32_t q_tok0;
    int32_t n_tok;
    int32_t kv_head;
    int32_t slot0;      // chunk c of this tile lives in slot slot0 + c
    int32_t n_chunks;
    int32_t request;
    int32_t reserved0;
    int32_t reserved1;
};
static_assert(sizeof(MergeItem) == 32, "MergeItem must stay 8 int32");

// Kernel arguments (passed by value).
struct TileArgs {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;            // may be null
    float *part_o;         // [slots][kTileRows][head_dim] fp32
    float *part_lse;       // [slots][kTileRows] fp32, base-2 log-sum-exp
    const Item *items;
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t group;         // num_qo_heads / num_kv_heads
    int32_t causal;
    float scale_log2;      // sm_scale * log2(e)
    // paged K/V (the paged kernel only): k and v are page pools
    // [pages][page_size][num_kv_heads][head_dim]; key j of request b sits in
    // page max(block_table[b * max_blocks + j / page_size], 0), slot j % page_size
    const int32_t *block_table;
    int32_t max_blocks;
    int32_t page_shift;    // log2(page_size)
    // FP8 K/V (the fp8 kernel only): k and v hold e4m3 bytes; O is scaled by
    // v_scale (k_scale is folded into scale_log2 by the host)
    float v_scale;
};

struct MergeArgs {
    void *o;
    float *lse;
    const float *part_o;
    const float *part_lse;
    const MergeItem *items;
    int32_t num_qo_heads;
    int32_t group;
};

// Host-side launchers (defined in the .hip file).  Return a hipError_t value.
// fold: the plan has fold items (launches the instance that runs them)
int launch_tile_kernel(int head_dim, bool paged, bool fp8, bool fold, const TileArgs &args,
                       int64_t num_items, void *stream);
int launch_tile_fold_kernel(int head_dim, bool paged, bool fp8, const TileArgs &args, int64_t num_items,
                            void *stream);
int launch_merge_kernel(int head_dim, const MergeArgs &args, int64_t num_items, void *stream);

}  // namespace rp
