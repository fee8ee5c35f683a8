// C ABI of the ragged prefill attention library: validation, plan/run,
// workspace management, status codes and logging.  Declared in
// include/ragged_prefill.h, which states the contract of every entry point.
#include "ragged_prefill.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <list>
#include <mutex>
#include <string>
#include <vector>

#include "rp_api_internal.h"
#include "rp_internal.h"
#include "rp_plan.h"
#include "rp_state_merge.h"

struct rp_plan {
    rp::HostPlan host;
    int device = -1;
    rp::Item *d_items = nullptr;
    rp::MergeItem *d_merges = nullptr;
    bool host_only = false;
    // Shared-prefix plans: `host` is the per-request (unique) level and
    // `shared` the level of all query rows against the shared prefix.
    rp_plan *shared = nullptr;
    int64_t q_begin = 0, q_end = 0;  // query rows both levels cover
};

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string &msg)
{
    g_last_error = msg;
    return status;
}

// ---- logging: RP_LOGLEVEL (0 off, 1 plans, 3 launches), RP_LOGDEST (stderr, stdout or a path)
int log_level()
{
    static int level = [] {
        const char *s = std::getenv("RP_LOGLEVEL");
        return s ? std::atoi(s) : 0;
    }();
    return level;
}

FILE *log_file()
{
    static FILE *f = [] {
        const char *d = std::getenv("RP_LOGDEST");
        if (d == nullptr || std::strcmp(d, "stderr") == 0)
            return stderr;
        if (std::strcmp(d, "stdout") == 0)
            return stdout;
        FILE *x = std::fopen(d, "a");
        return x ? x : stderr;
    }();
    return f;
}

void logf(int level, const char *fmt, ...)
{
    if (log_level() < level)
        return;
    FILE *f = log_file();
    std::fprintf(f, "[ragged_prefill] ");
    va_list ap;
    va_start(ap, fmt);
    std::vfprintf(f, fmt, ap);
    va_end(ap);
    std::fprintf(f, "\n");
    std::fflush(f);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Every device allocation of the library goes through here.  With
// RP_FAULT_INJECT=alloc in the environment (read at each call) it fails as an
// exhausted device would, which lets tests drive the RP_ENOMEM paths.
hipError_t device_alloc(void **p, size_t n)
{
    const char *f = std::getenv("RP_FAULT_INJECT");
    if (f != nullptr && std::strcmp(f, "alloc") == 0) {
        *p = nullptr;
        return hipErrorOutOfMemory;
    }
    return hipMalloc(p, n);
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(RP_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

int upload_plan(rp_plan *p)
{
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (!p->host.items.empty()) {
        const size_t n = p->host.items.size() * sizeof(rp::Item);
        e = device_alloc(reinterpret_cast<void **>(&p->d_items), n);
        if (e != hipSuccess)
            return fail(RP_ENOMEM, std::string("hipMalloc(worklist): ") + hipGetErrorString(e));
        e = hipMemcpy(p->d_items, p->host.items.data(), n, hipMemcpyHostToDevice);
        if (e != hipSuccess)
            return hip_fail(e, "hipMemcpy(worklist)");
    }
    if (!p->host.merges.empty()) {
        const size_t n = p->host.merges.size() * sizeof(rp::MergeItem);
        e = device_alloc(reinterpret_cast<void **>(&p->d_merges), n);
        if (e != hipSuccess)
            return fail(RP_ENOMEM, std::string("hipMalloc(merge list): ") + hipGetErrorString(e));
        e = hipMemcpy(p->d_merges, p->host.merges.data(), n, hipMemcpyHostToDevice);
        if (e != hipSuccess)
            return hip_fail(e, "hipMemcpy(merge list)");
    }
    return RP_OK;
}

void free_plan(rp_plan *p)
{
    if (p == nullptr)
        return;
    free_plan(p->shared);
    if (p->d_items)
        (void)hipFree(p->d_items);
    if (p->d_merges)
        (void)hipFree(p->d_merges);
    delete p;
}

int create_plan(const int32_t *q_indptr, const int32_t *kv_indptr, int batch, int num_qo_heads,
                int num_kv_heads, int head_dim, int causal, const rp_plan_opts *opts,
                rp_plan **out)
{
    if (out == nullptr)
        return fail(RP_EINVAL, "out must not be NULL");
    *out = nullptr;
    rp::PlanShape shape;
    shape.batch = batch;
    shape.num_qo_heads = num_qo_heads;
    shape.num_kv_heads = num_kv_heads;
    shape.head_dim = head_dim;
    shape.causal = causal ? 1 : 0;
    shape.kv_chunk = opts ? opts->kv_chunk : 0;
    shape.split_mode = opts ? opts->split_mode : 0;
    shape.num_xcds = opts ? opts->num_xcds : 0;
    rp_plan *p = new (std::nothrow) rp_plan;
    if (p == nullptr)
        return fail(RP_ENOMEM, "out of host memory");
    std::string err;
    int st;
    try {
        st = rp::build_plan(q_indptr, kv_indptr, shape, p->host, err);
    } catch (const std::bad_alloc &) {
        delete p;
        return fail(RP_ENOMEM, "out of host memory while planning");
    }
    if (st != RP_OK) {
        delete p;
        return fail(st, err);
    }
    p->host_only = opts && opts->host_only;
    if (!p->host_only) {
        st = upload_plan(p);
        if (st != RP_OK) {
            free_plan(p);
            return st;
        }
    }
    logf(1, "plan: batch=%d Hq=%d Hkv=%d D=%d causal=%d total_q=%lld total_kv=%lld items=%zu "
            "partial=%lld fold=%lld merges=%zu kv_chunk=%d gflop=%.3f mb=%.3f",
         batch, num_qo_heads, num_kv_heads, head_dim, causal, (long long)p->host.total_q,
         (long long)p->host.total_kv, p->host.items.size(), (long long)p->host.num_partial_items,
         (long long)p->host.num_fold_items, p->host.merges.size(), p->host.shape.kv_chunk, p->host.flops * 1e-9, p->host.bytes * 1e-6);
    *out = p;
    return RP_OK;
}

// Workspace layout of a shared-prefix plan (offsets in bytes, 256-aligned):
// [level workspace: max of both levels] [shared-level O, bf16 rows x Hq x D]
// [shared-level LSE, fp32 rows x Hq] [unique-level LSE, fp32 q_end x Hq].
struct SharedLayout {
    size_t o_shared, lse_shared, lse_unique, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

SharedLayout shared_layout(const rp_plan *p)
{
    const rp::PlanShape &sh = p->host.shape;
    const size_t rows = (size_t)(p->q_end - p->q_begin);
    SharedLayout L;
    const size_t level = std::max(p->host.workspace_bytes(), p->shared->host.workspace_bytes());
    L.o_shared = align256(level);
    L.lse_shared = L.o_shared + align256(rows * sh.num_qo_heads * sh.head_dim * 2);
    L.lse_unique = L.lse_shared + align256(rows * sh.num_qo_heads * 4);
    L.total = L.lse_unique + align256((size_t)p->q_end * sh.num_qo_heads * 4);
    return L;
}

size_t plan_workspace_bytes(const rp_plan *p)
{
    if (p == nullptr)
        return 0;
    return p->shared ? shared_layout(p).total : p->host.workspace_bytes();
}

// Validation of the state arrays of the merge entry points.
int check_merge_shape(int64_t rows, int num_heads, int head_dim)
{
    if (rows < 0 || num_heads <= 0 || num_heads > 0xffff)
        return fail(RP_EINVAL, "rows must be >= 0 and num_heads in [1, 65535]");
    if (head_dim < 8 || head_dim > 512 || (head_dim & (head_dim - 1)) != 0)
        return fail(RP_EINVAL, "head_dim must be a power of two in [8, 512]");
    return RP_OK;
}

int launch_merge(const rp::StateMergeArgs &a, void *stream)
{
    const int st = rp::launch_state_merge(a, stream);
    if (st != (int)hipSuccess)
        return hip_fail((hipError_t)st, "state merge kernel launch");
    return RP_OK;
}

// Paged K/V of one run (null: contiguous ragged K/V).
struct PagedKV {
    const int32_t *block_table;
    int max_blocks;
    int page_size;
};

// FP8 (e4m3) K/V of one run (null: bf16 K/V): dequantised value = code x scale.
struct Fp8KV {
    float k_scale;
    float v_scale;
};

int run_plan(const rp_plan *p, const void *q, const void *k, const void *v, void *o, float *lse,
             float sm_scale, void *workspace, size_t workspace_bytes, void *stream,
             const PagedKV *paged = nullptr, bool shared_level_call = false,
             const Fp8KV *fp8 = nullptr)
{
    if (p == nullptr)
        return fail(RP_EINVAL, "plan must not be NULL");
    if (p->host_only)
        return fail(RP_EINVAL, "a host-only plan cannot be run");
    if (p->shared && !shared_level_call)
        return fail(RP_EINVAL, "a shared-prefix plan runs through rp_run_shared_prefix");
    if (!std::isfinite(sm_scale))
        return fail(RP_EINVAL, "sm_scale must be finite");
    const rp::HostPlan &h = p->host;
    if (fp8) {
        if (!std::isfinite(fp8->k_scale) || !std::isfinite(fp8->v_scale))
            return fail(RP_EINVAL, "k_scale and v_scale must be finite");
    }
    if (h.items.empty())
        return RP_OK;  // empty batch / no query rows: nothing to launch
    if (q == nullptr || o == nullptr)
        return fail(RP_EINVAL, "q and o must not be NULL");
    if (h.total_kv > 0 && (k == nullptr || v == nullptr))
        return fail(RP_EINVAL, "k and v must not be NULL");
    if (!aligned16(q) || !aligned16(o) || !aligned16(k) || !aligned16(v) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
        return fail(RP_EINVAL, "q, k, v and o must be 16-byte aligned (lse 4-byte)");
    int page_shift = 0;
    if (paged) {
        const int ps = paged->page_size;
        if (ps != 16 && ps != 32 && ps != 64 && ps != 128)
            return fail(RP_EINVAL, "page_size must be 16, 32, 64 or 128");
        while ((1 << page_shift) < ps)
            ++page_shift;
        int64_t max_kv = 0;
        for (const rp::Item &it : h.items)
            max_kv = std::max<int64_t>(max_kv, it.kv_len);
        const int64_t need_blocks = (max_kv + ps - 1) / ps;
        if (paged->max_blocks < need_blocks)
            return fail(RP_EINVAL, "max_blocks_per_seq " + std::to_string(paged->max_blocks) +
                                       " is below the " + std::to_string(need_blocks) +
                                       " pages the longest request needs");
        if (max_kv > 0 && paged->block_table == nullptr)
            return fail(RP_EINVAL, "block_table must not be NULL");
        if ((reinterpret_cast<uintptr_t>(paged->block_table) & 3u) != 0)
            return fail(RP_EINVAL, "block_table must be 4-byte aligned");
    }
    const size_t need = h.workspace_bytes();
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes < need)
            return fail(RP_EINVAL, "workspace too small: need " + std::to_string(need) + " bytes");
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(RP_EINVAL, "workspace must be 256-byte aligned");
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev != p->device)
        return fail(RP_EINVAL, "plan was created on device " + std::to_string(p->device) +
                                   " but device " + std::to_string(dev) + " is current");

    float *part_o = static_cast<float *>(workspace);
    float *part_lse = need ? reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                                       ((h.part_o_bytes() + 255) & ~size_t(255)))
                           : nullptr;
    rp::TileArgs ta{};
    ta.q = q;
    ta.k = k;
    ta.v = v;
    ta.o = o;
    ta.lse = lse;
    ta.part_o = part_o;
    ta.part_lse = part_lse;
    ta.items = p->d_items;
    ta.num_qo_heads = h.shape.num_qo_heads;
    ta.num_kv_heads = h.shape.num_kv_heads;
    ta.group = h.shape.num_qo_heads / h.shape.num_kv_heads;
    ta.causal = h.shape.causal;
    ta.scale_log2 = (float)((double)sm_scale * (fp8 ? (double)fp8->k_scale : 1.0) * 1.4426950408889634);
    ta.v_scale = fp8 ? fp8->v_scale : 1.0f;
    if (paged) {
        ta.block_table = paged->block_table;
        ta.max_blocks = paged->max_blocks;
        ta.page_shift = page_shift;
    }
    logf(3, "launch tile kernel: D=%d items=%zu merges=%zu scale_log2=%g", h.shape.head_dim,
         h.items.size(), h.merges.size(), (double)ta.scale_log2);
    int st = rp::launch_tile_kernel(h.shape.head_dim, paged != nullptr, fp8 != nullptr,
                                    h.num_fold_items > 0, ta, (int64_t)h.items.size(), stream);
    if (st != (int)hipSuccess)
        return hip_fail((hipError_t)st, "tile kernel launch");
    if (!h.merges.empty()) {
        rp::MergeArgs ma{};
        ma.o = o;
        ma.lse = lse;
        ma.part_o = part_o;
        ma.part_lse = part_lse;
        ma.items = p->d_merges;
        ma.num_qo_heads = h.shape.num_qo_heads;
        ma.group = ta.group;
        st = rp::launch_merge_kernel(h.shape.head_dim, ma, (int64_t)h.merges.size(), stream);
        if (st != (int)hipSuccess)
            return hip_fail((hipError_t)st, "merge kernel launch");
    }
    return RP_OK;
}

// ---- one-shot path: per-device plan cache and library-owned workspace ----
struct CachedPlan {
    std::vector<int32_t> q_indptr, kv_indptr;
    int num_qo_heads, num_kv_heads, head_dim, causal;
    rp_plan *plan;
};

// Split-KV workspace of one stream (partial states are written by the tile
// kernel and read by the merge kernel of the same call, so calls on one
// stream may share it; calls on different streams may not).
struct StreamWorkspace {
    void *stream;
    void *ptr = nullptr;
    size_t bytes = 0;
};

struct DeviceState {
    std::list<CachedPlan> plans;             // most recent first
    std::list<StreamWorkspace> workspaces;   // most recent first
};

constexpr size_t kPlanCacheSize = 8;
constexpr size_t kStreamCacheSize = 8;
std::mutex g_oneshot_mutex;
// Cached plans and workspaces live until the process ends.  The holder is
// never destroyed, so nothing is freed during static destruction (when the
// HIP runtime may already be gone) and the memory stays reachable.
std::vector<DeviceState> &device_states()
{
    static auto *states = new std::vector<DeviceState>();
    return *states;
}

}  // namespace

namespace rp {

int record_error(int status, const char *msg) { return fail(status, msg); }

int run_plan_on(const rp_plan *plan, const void *q, const void *k, const void *v, void *o,
                float *lse, float sm_scale, void *workspace, size_t workspace_bytes,
                void *stream)
{
    return run_plan(plan, q, k, v, o, lse, sm_scale, workspace, workspace_bytes, stream);
}

}  // namespace rp

extern "C" {

const char *rp_status_string(int status)
{
    switch (status) {
    case RP_OK: return "RP_OK";
    case RP_EINVAL: return "RP_EINVAL: invalid argument";
    case RP_EUNSUPPORTED: return "RP_EUNSUPPORTED: unsupported configuration";
    case RP_ENOMEM: return "RP_ENOMEM: out of memory";
    case RP_EDEVICE: return "RP_EDEVICE: HIP runtime or launch failure";
    default: return "unknown status";
    }
}

const char *rp_last_error(void) { return g_last_error.c_str(); }

int rp_abi_version(void) { return RP_ABI_VERSION; }

int rp_available(void)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return 0;
    return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

int rp_plan_create(const int32_t *q_indptr, const int32_t *kv_indptr, int batch, int num_qo_heads,
                   int num_kv_heads, int head_dim, int causal, const rp_plan_opts *opts,
                   rp_plan **out)
{
    return create_plan(q_indptr, kv_indptr, batch, num_qo_heads, num_kv_heads, head_dim, causal,
                       opts, out);
}

int rp_plan_get_info(const rp_plan *p, rp_plan_info *info)
{
    if (p == nullptr || info == nullptr)
        return fail(RP_EINVAL, "plan and info must not be NULL");
    const rp::HostPlan &h = p->host;
    std::memset(info, 0, sizeof *info);
    info->num_items = (int64_t)h.items.size();
    info->num_partial_items = h.num_partial_items;
    info->num_merge_items = (int64_t)h.merges.size();
    info->num_fold_items = h.num_fold_items;
    info->total_q = h.total_q;
    info->total_kv = h.total_kv;
    info->tile_rows = rp::kTileRows;
    info->tile_tokens = h.tile_tokens;
    info->key_block = rp::key_block(h.shape.head_dim);
    info->kv_chunk = h.shape.kv_chunk;
    info->flops = h.flops;
    info->bytes = h.bytes;
    if (p->shared) {
        // both levels; algorithmic bytes add the shared K and V, read once
        const rp::HostPlan &s = p->shared->host;
        info->num_items += (int64_t)s.items.size();
        info->num_partial_items += s.num_partial_items;
        info->num_merge_items += (int64_t)s.merges.size();
        info->num_fold_items += s.num_fold_items;
        info->total_kv += s.total_kv;
        info->flops += s.flops;
        info->bytes += 2.0 * 2.0 * (double)s.total_kv * h.shape.num_kv_heads * h.shape.head_dim;
    }
    info->workspace_bytes = plan_workspace_bytes(p);
    return RP_OK;
}

size_t rp_plan_workspace_bytes(const rp_plan *p) { return plan_workspace_bytes(p); }

int64_t rp_plan_copy_items(const rp_plan *p, int32_t *dst, int64_t capacity)
{
    if (p == nullptr || (dst == nullptr && capacity > 0) || capacity < 0)
        return fail(RP_EINVAL, "bad arguments");
    const int64_t n = std::min<int64_t>(capacity, (int64_t)p->host.items.size());
    if (n > 0)
        std::memcpy(dst, p->host.items.data(), (size_t)n * sizeof(rp::Item));
    return n;
}

int rp_run(const rp_plan *p, const void *q, const void *k, const void *v, void *o, float *lse,
           float sm_scale, void *workspace, size_t workspace_bytes, void *stream)
{
    return run_plan(p, q, k, v, o, lse, sm_scale, workspace, workspace_bytes, stream);
}

int rp_run_paged(const rp_plan *p, const void *q, const void *k_pages, const void *v_pages,
                 const int32_t *block_table, int max_blocks_per_seq, int page_size, void *o,
                 float *lse, float sm_scale, void *workspace, size_t workspace_bytes, void *stream)
{
    PagedKV pk{block_table, max_blocks_per_seq, page_size};
    return run_plan(p, q, k_pages, v_pages, o, lse, sm_scale, workspace, workspace_bytes, stream, &pk);
}

int rp_run_fp8kv(const rp_plan *p, const void *q, const void *k_fp8, const void *v_fp8, float k_scale,
                 float v_scale, void *o, float *lse, float sm_scale, void *workspace,
                 size_t workspace_bytes, void *stream)
{
    Fp8KV f{k_scale, v_scale};
    return run_plan(p, q, k_fp8, v_fp8, o, lse, sm_scale, workspace, workspace_bytes, stream, nullptr,
                    false, &f);
}

int rp_run_paged_fp8kv(const rp_plan *p, const void *q, const void *k_pages, const void *v_pages,
                       const int32_t *block_table, int max_blocks_per_seq, int page_size,
                       float k_scale, float v_scale, void *o, float *lse, float sm_scale,
                       void *workspace, size_t workspace_bytes, void *stream)
{
    PagedKV pk{block_table, max_blocks_per_seq, page_size};
    Fp8KV f{k_scale, v_scale};
    return run_plan(p, q, k_pages, v_pages, o, lse, sm_scale, workspace, workspace_bytes, stream, &pk,
                    false, &f);
}

void rp_plan_destroy(rp_plan *p) { free_plan(p); }

int rp_plan_create_shared_prefix(const int32_t *q_indptr, const int32_t *kv_indptr, int batch,
                                 int shared_kv_len, int num_qo_heads, int num_kv_heads,
                                 int head_dim, int causal, const rp_plan_opts *opts, rp_plan **out)
{
    if (out == nullptr)
        return fail(RP_EINVAL, "out must not be NULL");
    *out = nullptr;
    if (shared_kv_len < 0)
        return fail(RP_EINVAL, "shared_kv_len must be >= 0");
    if (batch < 0 || (batch > 0 && (q_indptr == nullptr || kv_indptr == nullptr)))
        return fail(RP_EINVAL, "batch must be >= 0 and the offsets non-NULL");
    if (causal) {
        // Bottom-right causal over [prefix, own keys] shows the whole prefix to
        // every row only if no request has more queries than own keys.
        for (int b = 0; b < batch; ++b) {
            const int64_t qo = (int64_t)q_indptr[b + 1] - q_indptr[b];
            const int64_t kv = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
            if (qo > kv && shared_kv_len > 0)
                return fail(RP_EINVAL, "causal shared-prefix attention needs qo_len <= kv_len "
                                       "in every request (request " + std::to_string(b) + ")");
        }
    }
    rp_plan *unique = nullptr;
    int st = create_plan(q_indptr, kv_indptr, batch, num_qo_heads, num_kv_heads, head_dim, causal,
                         opts, &unique);
    if (st != RP_OK)
        return st;
    // the shared level: all query rows as one request over the prefix, no mask
    const int64_t q0 = batch > 0 ? q_indptr[0] : 0, q1 = batch > 0 ? q_indptr[batch] : 0;
    const int32_t sq[2] = {0, (int32_t)(q1 - q0)};
    const int32_t skv[2] = {0, shared_kv_len};
    rp_plan *shared = nullptr;
    st = create_plan(sq, skv, 1, num_qo_heads, num_kv_heads, head_dim, 0, opts, &shared);
    if (st != RP_OK) {
        free_plan(unique);
        return st;
    }
    unique->shared = shared;
    unique->q_begin = q0;
    unique->q_end = q1;
    *out = unique;
    return RP_OK;
}

namespace {

// Shared-prefix attention: the shared level, the own-key level (contiguous
// or paged K/V), then the in-place merge of the two states.
int run_shared_prefix(const rp_plan *p, const void *q, const void *k_shared, const void *v_shared,
                      const void *k_own, const void *v_own, const PagedKV *paged, void *o,
                      float *lse, float sm_scale, void *workspace, size_t workspace_bytes,
                      void *stream)
{
    if (p == nullptr || p->shared == nullptr)
        return fail(RP_EINVAL, "plan must come from rp_plan_create_shared_prefix");
    if (p->host_only)
        return fail(RP_EINVAL, "a host-only plan cannot be run");
    if (p->q_end == p->q_begin)
        return RP_OK;
    if (q == nullptr || o == nullptr)
        return fail(RP_EINVAL, "q and o must not be NULL");
    const SharedLayout L = shared_layout(p);
    if (workspace == nullptr || workspace_bytes < L.total)
        return fail(RP_EINVAL, "workspace too small: need " + std::to_string(L.total) + " bytes");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(RP_EINVAL, "workspace must be 256-byte aligned");
    const rp::PlanShape &sh = p->host.shape;
    char *ws = static_cast<char *>(workspace);
    const size_t row_elems = (size_t)sh.num_qo_heads * sh.head_dim;
    const size_t row_bytes = row_elems * 2;  // bf16
    const void *q_rows = static_cast<const char *>(q) + (size_t)p->q_begin * row_bytes;
    void *o_shared = ws + L.o_shared;
    float *lse_shared = reinterpret_cast<float *>(ws + L.lse_shared);
    float *lse_unique = reinterpret_cast<float *>(ws + L.lse_unique);
    // 1. every query row against the shared prefix (one request, no mask)
    int st = run_plan(p->shared, q_rows, k_shared, v_shared, o_shared, lse_shared, sm_scale, ws,
                      L.o_shared, stream, nullptr, true);
    if (st != RP_OK)
        return st;
    // 2. each request against its own keys, into o
    st = run_plan(p, q, k_own, v_own, o, lse_unique, sm_scale, ws, L.o_shared, stream, paged, true);
    if (st != RP_OK)
        return st;
    // 3. o, lse = merge(shared state, own state), in place over o
    rp::StateMergeArgs a{};
    a.v0 = o_shared;
    a.s0 = lse_shared;
    a.v1 = static_cast<char *>(o) + (size_t)p->q_begin * row_bytes;
    a.s1 = lse_unique + (size_t)p->q_begin * sh.num_qo_heads;
    a.v_out = const_cast<void *>(a.v1);
    a.s_out = lse ? lse + (size_t)p->q_begin * sh.num_qo_heads : nullptr;
    a.v_row_stride = (int64_t)row_elems;
    a.s_row_stride = sh.num_qo_heads;
    a.rows = p->q_end - p->q_begin;
    a.num_heads = sh.num_qo_heads;
    a.head_dim = sh.head_dim;
    a.num_states = 2;
    return launch_merge(a, stream);
}

}  // namespace

int rp_run_shared_prefix(const rp_plan *p, const void *q, const void *k_shared,
                         const void *v_shared, const void *k_unique, const void *v_unique, void *o,
                         float *lse, float sm_scale, void *workspace, size_t workspace_bytes,
                         void *stream)
{
    return run_shared_prefix(p, q, k_shared, v_shared, k_unique, v_unique, nullptr, o, lse,
                             sm_scale, workspace, workspace_bytes, stream);
}

int rp_run_shared_prefix_paged(const rp_plan *p, const void *q, const void *k_shared,
                               const void *v_shared, const void *k_pages, const void *v_pages,
                               const int32_t *block_table, int max_blocks_per_seq, int page_size,
                               void *o, float *lse, float sm_scale, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    PagedKV pk{block_table, max_blocks_per_seq, page_size};
    return run_shared_prefix(p, q, k_shared, v_shared, k_pages, v_pages, &pk, o, lse, sm_scale,
                             workspace, workspace_bytes, stream);
}

int rp_merge_state(const void *v_a, const float *s_a, const void *v_b, const float *s_b,
                   void *v_out, float *s_out, int64_t rows, int num_heads, int head_dim,
                   void *stream)
{
    int st = check_merge_shape(rows, num_heads, head_dim);
    if (st != RP_OK)
        return st;
    if (rows == 0)
        return RP_OK;
    if (!v_a || !s_a || !v_b || !s_b || !v_out)
        return fail(RP_EINVAL, "v_a, s_a, v_b, s_b and v_out must not be NULL");
    if (!aligned16(v_a) || !aligned16(v_b) || !aligned16(v_out))
        return fail(RP_EINVAL, "v_a, v_b and v_out must be 16-byte aligned");
    rp::StateMergeArgs a{};
    a.v0 = v_a;
    a.v1 = v_b;
    a.s0 = s_a;
    a.s1 = s_b;
    a.v_out = v_out;
    a.s_out = s_out;
    a.v_row_stride = (int64_t)num_heads * head_dim;
    a.s_row_stride = num_heads;
    a.rows = rows;
    a.num_heads = num_heads;
    a.head_dim = head_dim;
    a.num_states = 2;
    return launch_merge(a, stream);
}

int rp_merge_state_in_place(void *v, float *s, const void *v_other, const float *s_other,
                            int64_t rows, int num_heads, int head_dim, void *stream)
{
    if (s == nullptr)
        return fail(RP_EINVAL, "s must not be NULL");
    return rp_merge_state(v, s, v_other, s_other, v, s, rows, num_heads, head_dim, stream);
}

int rp_merge_states(const void *v, const float *s, void *v_out, float *s_out, int64_t rows,
                    int num_states, int num_heads, int head_dim, void *stream)
{
    int st = check_merge_shape(rows, num_heads, head_dim);
    if (st != RP_OK)
        return st;
    if (num_states < 1)
        return fail(RP_EINVAL, "num_states must be >= 1");
    if (rows == 0)
        return RP_OK;
    if (!v || !s || !v_out)
        return fail(RP_EINVAL, "v, s and v_out must not be NULL");
    if (!aligned16(v) || !aligned16(v_out))
        return fail(RP_EINVAL, "v and v_out must be 16-byte aligned");
    rp::StateMergeArgs a{};
    a.v0 = v;
    a.s0 = s;
    a.v_out = v_out;
    a.s_out = s_out;
    a.v_state_stride = (int64_t)num_heads * head_dim;
    a.v_row_stride = (int64_t)num_states * num_heads * head_dim;
    a.s_state_stride = num_heads;
    a.s_row_stride = (int64_t)num_states * num_heads;
    a.rows = rows;
    a.num_heads = num_heads;
    a.head_dim = head_dim;
    a.num_states = num_states;
    return launch_merge(a, stream);
}

int ragged_prefill_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                        const int32_t *q_indptr, const int32_t *kv_indptr, int batch,
                        int num_qo_heads, int num_kv_heads, int head_dim, int causal,
                        float sm_scale, void *stream)
{
    if (batch < 0)
        return fail(RP_EINVAL, "batch must be >= 0");
    if (batch == 0)
        return RP_OK;  // empty batch: early return, no launch
    if (q_indptr == nullptr || kv_indptr == nullptr)
        return fail(RP_EINVAL, "q_indptr and kv_indptr must not be NULL");
    if (!std::isfinite(sm_scale))
        return fail(RP_EINVAL, "sm_scale must be finite");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(static_cast<hipStream_t>(stream), &capture);
    if (e != hipSuccess)
        return hip_fail(e, "hipStreamIsCapturing");
    const bool capturing = capture != hipStreamCaptureStatusNone;
    std::lock_guard<std::mutex> lock(g_oneshot_mutex);
    std::vector<DeviceState> &devices = device_states();
    if ((int)devices.size() <= dev)
        devices.resize((size_t)dev + 1);
    DeviceState &ds = devices[(size_t)dev];
    const int cz = causal ? 1 : 0;
    rp_plan *plan = nullptr;
    for (auto it = ds.plans.begin(); it != ds.plans.end(); ++it) {
        if (it->num_qo_heads == num_qo_heads && it->num_kv_heads == num_kv_heads &&
            it->head_dim == head_dim && it->causal == cz &&
            (int)it->q_indptr.size() == batch + 1 &&
            std::memcmp(it->q_indptr.data(), q_indptr, sizeof(int32_t) * (batch + 1)) == 0 &&
            std::memcmp(it->kv_indptr.data(), kv_indptr, sizeof(int32_t) * (batch + 1)) == 0) {
            plan = it->plan;
            ds.plans.splice(ds.plans.begin(), ds.plans, it);
            break;
        }
    }
    if (plan == nullptr) {
        if (capturing)
            return fail(RP_EINVAL, "one-shot call under graph capture needs a cached plan: "
                                   "call once with these offsets outside the capture first");
        int st = create_plan(q_indptr, kv_indptr, batch, num_qo_heads, num_kv_heads, head_dim, cz,
                             nullptr, &plan);
        if (st != RP_OK)
            return st;
        CachedPlan cp;
        cp.q_indptr.assign(q_indptr, q_indptr + batch + 1);
        cp.kv_indptr.assign(kv_indptr, kv_indptr + batch + 1);
        cp.num_qo_heads = num_qo_heads;
        cp.num_kv_heads = num_kv_heads;
        cp.head_dim = head_dim;
        cp.causal = cz;
        cp.plan = plan;
        ds.plans.push_front(std::move(cp));
        while (ds.plans.size() > kPlanCacheSize) {
            // the evicted plan's worklist may still be read by queued work on any stream
            (void)hipDeviceSynchronize();
            free_plan(ds.plans.back().plan);
            ds.plans.pop_back();
        }
    }
    const size_t need = plan->host.workspace_bytes();
    void *ws = nullptr;
    size_t ws_bytes = 0;
    if (need > 0) {
        auto it = ds.workspaces.begin();
        for (; it != ds.workspaces.end(); ++it)
            if (it->stream == stream)
                break;
        if (it != ds.workspaces.end())
            ds.workspaces.splice(ds.workspaces.begin(), ds.workspaces, it);
        else
            ds.workspaces.push_front(StreamWorkspace{stream});
        StreamWorkspace &sw = ds.workspaces.front();
        if (need > sw.bytes) {
            if (capturing)
                return fail(RP_EINVAL, "one-shot call under graph capture needs this stream's "
                                       "workspace to be large enough: call once with these "
                                       "offsets on this stream outside the capture first");
            if (sw.ptr) {
                // queued work of this stream may still use the old workspace
                e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
                if (e != hipSuccess)
                    return hip_fail(e, "hipStreamSynchronize");
                (void)hipFree(sw.ptr);
                sw.ptr = nullptr;
                sw.bytes = 0;
            }
            e = device_alloc(&sw.ptr, need);
            if (e != hipSuccess) {
                sw.ptr = nullptr;
                return fail(RP_ENOMEM, std::string("hipMalloc(workspace): ") + hipGetErrorString(e));
            }
            sw.bytes = need;
        }
        ws = sw.ptr;
        ws_bytes = sw.bytes;
        while (ds.workspaces.size() > kStreamCacheSize) {
            // the evicted stream may have been destroyed: wait for the whole device
            (void)hipDeviceSynchronize();
            if (ds.workspaces.back().ptr)
                (void)hipFree(ds.workspaces.back().ptr);
            ds.workspaces.pop_back();
        }
    }
    return run_plan(plan, q, k, v, o, lse, sm_scale, ws, ws_bytes, stream);
}

}  // extern "C"
