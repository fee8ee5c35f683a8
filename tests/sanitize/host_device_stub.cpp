// Host-only stand-in for the device side of the library, for the sanitizer
// build of the planner and the C ABI (tests/test_sanitize_cpu.py).
//
// The HIP runtime calls the ABI makes are replaced by host equivalents:
// "device memory" is host memory from malloc, copies are memcpy, there is one
// device (0) and no stream is ever capturing.  The kernel launchers are
// replaced by functions that walk the launch's work list and touch every byte
// range the kernel would read or write (first and last byte of each row
// slice), so that AddressSanitizer reports any range that reaches outside the
// buffers the test allocated with exactly the documented sizes.  Nothing is
// computed.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "rp_internal.h"
#include "rp_state_merge.h"

namespace {

volatile unsigned char g_sink;

void touch_read(const void *p, size_t bytes)
{
    if (bytes == 0)
        return;
    const unsigned char *c = static_cast<const unsigned char *>(p);
    g_sink = c[0];
    g_sink = c[bytes - 1];
}

void touch_write(void *p, size_t bytes)
{
    if (bytes == 0)
        return;
    unsigned char *c = static_cast<unsigned char *>(p);
    c[0] = 0;
    c[bytes - 1] = 0;
}

[[noreturn]] void contract(const char *what, long long a, long long b)
{
    std::fprintf(stderr, "launch contract violated: %s (%lld, %lld)\n", what, a, b);
    std::abort();
}

}  // namespace

extern "C" {

hipError_t hipMalloc(void **ptr, size_t size)
{
    *ptr = std::malloc(size ? size : 1);
    return *ptr ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipFree(void *ptr)
{
    std::free(ptr);
    return hipSuccess;
}

hipError_t hipMemcpy(void *dst, const void *src, size_t bytes, hipMemcpyKind)
{
    std::memcpy(dst, src, bytes);
    return hipSuccess;
}

hipError_t hipGetDevice(int *device)
{
    *device = 0;
    return hipSuccess;
}

hipError_t hipDeviceSynchronize(void) { return hipSuccess; }

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus *status)
{
    *status = hipStreamCaptureStatusNone;
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t) { return "host stand-in error"; }

hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *, int) { return hipErrorNoDevice; }

}  // extern "C"

namespace rp {

int launch_tile_fold_kernel(int, bool, bool, const TileArgs &, int64_t, void *)
{
    contract("fold launcher called directly", 0, 0);
}

int launch_tile_kernel(int head_dim, bool paged, bool fp8, bool fold, const TileArgs &a,
                       int64_t num_items, void *)
{
    const int g = a.group;
    const size_t elem = fp8 ? 1 : 2;   // K/V bytes per element
    const size_t q_row = (size_t)a.num_qo_heads * head_dim * 2;
    const size_t kv_row = (size_t)a.num_kv_heads * head_dim * elem;
    for (int64_t i = 0; i < num_items; ++i) {
        const Item &it = a.items[i];
        if (it.n_tok == 0)
            continue;
        if (it.n_tok < 0 || it.n_tok * g > kTileRows || it.t0 < 0 || it.t0 + it.n_tok > it.qo_len)
            contract("tile token range", it.t0, it.n_tok);
        if (it.kv_head < 0 || it.kv_head >= a.num_kv_heads)
            contract("kv head", it.kv_head, a.num_kv_heads);
        // a fold item writes the final O/LSE and keeps its running state in its slot
        const bool fold_item = it.fold_keys > 0;
        if (fold_item && (!fold || it.slot < 0))
            contract("fold item in a launch without fold items", it.slot, fold ? 1 : 0);
        const bool keys = it.key_end > it.key_begin;
        if (keys && (it.key_begin < 0 || it.key_end > it.kv_len))
            contract("key range", it.key_begin, it.key_end);
        // Q rows of the tile (the g heads of the group), O and LSE of the same rows
        for (int t = 0; t < it.n_tok; ++t) {
            const size_t row = (size_t)it.q_tok0 + t;
            const size_t off = row * q_row + (size_t)it.kv_head * g * head_dim * 2;
            touch_read(static_cast<const char *>(a.q) + off, (size_t)g * head_dim * 2);
            if (it.slot < 0 || fold_item) {
                touch_write(static_cast<char *>(a.o) + off, (size_t)g * head_dim * 2);
                if (a.lse)
                    touch_write(a.lse + row * a.num_qo_heads + (size_t)it.kv_head * g, (size_t)g * 4);
            }
        }
        if (it.slot >= 0) {
            touch_write(a.part_o + (size_t)it.slot * kTileRows * head_dim, (size_t)kTileRows * head_dim * 4);
            touch_write(a.part_lse + (size_t)it.slot * kTileRows, (size_t)kTileRows * 4);
        }
        if (!keys)
            continue;
        // K and V rows: the request's keys key_begin..key_end-1 (the kernel
        // clamps a block's rows to the request's last key)
        for (int j = it.key_begin; j < it.key_end; ++j) {
            size_t off;
            if (paged) {
                const int page_size = 1 << a.page_shift;
                if (j / page_size >= a.max_blocks)
                    contract("block table column", j / page_size, a.max_blocks);
                const int32_t *entry = a.block_table + (size_t)it.request * a.max_blocks + j / page_size;
                touch_read(entry, 4);
                const int page = *entry < 0 ? 0 : *entry;
                off = ((size_t)page * page_size + (size_t)(j % page_size)) * kv_row;
            } else {
                off = ((size_t)it.kv_row0 + j) * kv_row;
            }
            off += (size_t)it.kv_head * head_dim * elem;
            touch_read(static_cast<const char *>(a.k) + off, (size_t)head_dim * elem);
            touch_read(static_cast<const char *>(a.v) + off, (size_t)head_dim * elem);
        }
    }
    return 0;
}

int launch_merge_kernel(int head_dim, const MergeArgs &a, int64_t num_items, void *)
{
    for (int64_t i = 0; i < num_items; ++i) {
        const MergeItem &it = a.items[i];
        if (it.n_chunks < 1 || it.n_tok < 1 || it.n_tok * a.group > kTileRows)
            contract("merge item", it.n_chunks, it.n_tok);
        for (int c = 0; c < it.n_chunks; ++c) {
            touch_read(a.part_o + ((size_t)it.slot0 + c) * kTileRows * head_dim, (size_t)kTileRows * head_dim * 4);
            touch_read(a.part_lse + ((size_t)it.slot0 + c) * kTileRows, (size_t)kTileRows * 4);
        }
        for (int t = 0; t < it.n_tok; ++t) {
            const size_t row = (size_t)it.q_tok0 + t;
            touch_write(static_cast<char *>(a.o) + (row * a.num_qo_heads + (size_t)it.kv_head * a.group) * head_dim * 2,
                        (size_t)a.group * head_dim * 2);
            if (a.lse)
                touch_write(a.lse + row * a.num_qo_heads + (size_t)it.kv_head * a.group, (size_t)a.group * 4);
        }
    }
    return 0;
}

int launch_state_merge(const StateMergeArgs &a, void *)
{
    const size_t vb = (size_t)a.head_dim * 2;
    for (int64_t r = 0; r < a.rows; ++r)
        for (int h = 0; h < a.num_heads; ++h) {
            for (int i = 0; i < a.num_states; ++i) {
                const char *v = (a.v1 && i == 1) ? static_cast<const char *>(a.v1)
                                                 : static_cast<const char *>(a.v0) + i * a.v_state_stride * 2;
                const float *s = (a.s1 && i == 1) ? a.s1 : a.s0 + i * a.s_state_stride;
                touch_read(v + (r * a.v_row_stride + (int64_t)h * a.head_dim) * 2, vb);
                touch_read(s + r * a.s_row_stride + h, 4);
            }
            touch_write(static_cast<char *>(a.v_out) + (r * a.num_heads + h) * vb, vb);
            if (a.s_out)
                touch_write(a.s_out + r * a.num_heads + h, 4);
        }
    return 0;
}

}  // namespace rp
