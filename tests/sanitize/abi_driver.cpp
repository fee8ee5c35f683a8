// Drives the C ABI (planner, plan/run, paged and FP8 runs, one-shot plan and
// workspace caches, shared prefix, state merges, argument validation and the
// injected allocation failure) over many seeded random batches, against the
// host stand-in of host_device_stub.cpp.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitize_cpu.py; every buffer has
// exactly its documented size, so any access beyond it is reported.
// Exit status 0 and "abi driver: ok" on success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ragged_prefill.h"

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;

uint32_t rnd()
{
    // xorshift64*
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (uint32_t)((g_state * 0x2545f4914f6cdd1dull) >> 32);
}

int fails = 0;

void expect(bool ok, const char *what, int iter)
{
    if (!ok) {
        std::fprintf(stderr, "iteration %d: %s (%s)\n", iter, what, rp_last_error());
        ++fails;
    }
}

struct Buf {
    void *p = nullptr;
    size_t n = 0;
    explicit Buf(size_t bytes, unsigned char fill = 0x5a) : n(bytes)
    {
        // 256-byte aligned (the workspace needs it), exactly `bytes` long
        if (posix_memalign(&p, 256, bytes ? bytes : 1) != 0)
            std::abort();
        std::memset(p, fill, bytes ? bytes : 1);
    }
    ~Buf() { std::free(p); }
    Buf(const Buf &) = delete;
    Buf &operator=(const Buf &) = delete;
};

struct Batch {
    int batch, hq, hkv, d, causal;
    std::vector<int32_t> qi, ki;
    int64_t rows_q, rows_kv;
};

Batch random_batch()
{
    static const int heads[][2] = {{4, 2}, {8, 2}, {8, 8}, {32, 8}, {12, 4}, {16, 1}, {64, 8}};
    Batch b;
    b.batch = (int)(rnd() % 10);
    const int h = (int)(rnd() % 7);
    b.hq = heads[h][0];
    b.hkv = heads[h][1];
    b.d = rnd() % 2 ? 128 : 256;
    b.causal = (int)(rnd() % 2);
    const int q0 = (int)(rnd() % 4), k0 = (int)(rnd() % 4);
    b.qi.push_back(q0);
    b.ki.push_back(k0);
    for (int r = 0; r < b.batch; ++r) {
        int qo, kv;
        switch (rnd() % 6) {
        case 0: qo = 0; kv = (int)(rnd() % 50); break;
        case 1: qo = 1; kv = (int)(rnd() % 3000); break;            // decode-like
        case 2: qo = (int)(rnd() % 300); kv = qo; break;
        case 3: qo = (int)(rnd() % 200); kv = qo + (int)(rnd() % 900); break;  // append
        case 4: qo = (int)(rnd() % 100) + 1; kv = (int)(rnd() % 3); break;    // qo > kv
        default: qo = (int)(rnd() % 64); kv = (int)(rnd() % 64); break;
        }
        b.qi.push_back(b.qi.back() + qo);
        b.ki.push_back(b.ki.back() + kv);
    }
    b.rows_q = b.qi.back();
    b.rows_kv = b.ki.back();
    return b;
}

void run_batch(const Batch &b, int iter)
{
    static const int chunks[] = {0, 64, 128, 192, 1024};
    rp_plan_opts opts{};
    opts.kv_chunk = chunks[rnd() % 5];
    static const int modes[] = {RP_SPLIT_AUTO, RP_SPLIT_NEVER, RP_SPLIT_ALWAYS};
    opts.split_mode = modes[rnd() % 3];
    opts.num_xcds = (int)(rnd() % 9);
    rp_plan *plan = nullptr;
    int st = rp_plan_create(b.qi.data(), b.ki.data(), b.batch, b.hq, b.hkv, b.d, b.causal, &opts, &plan);
    expect(st == RP_OK && plan != nullptr, "rp_plan_create", iter);
    if (st != RP_OK)
        return;
    rp_plan_info info;
    expect(rp_plan_get_info(plan, &info) == RP_OK, "rp_plan_get_info", iter);
    std::vector<int32_t> items((size_t)(info.num_items + 1) * RP_ITEM_INTS);
    expect(rp_plan_copy_items(plan, items.data(), info.num_items) == info.num_items, "copy items", iter);

    const size_t qb = (size_t)b.rows_q * b.hq * b.d * 2;
    const size_t kb = (size_t)b.rows_kv * b.hkv * b.d * 2;
    Buf q(qb), k(kb), v(kb), o(qb), lse((size_t)b.rows_q * b.hq * 4);
    const size_t wsb = rp_plan_workspace_bytes(plan);
    Buf ws(wsb);
    const float scale = 1.0f / std::sqrt((float)b.d);
    st = rp_run(plan, q.p, k.p, v.p, o.p, (float *)lse.p, scale, wsb ? ws.p : nullptr, wsb, nullptr);
    expect(st == RP_OK, "rp_run", iter);
    if (wsb > 0)
        expect(rp_run(plan, q.p, k.p, v.p, o.p, (float *)lse.p, scale, ws.p, wsb - 1, nullptr) == RP_EINVAL,
               "rp_run must refuse a short workspace", iter);
    expect(rp_run(plan, q.p, k.p, v.p, o.p, nullptr, NAN, ws.p, wsb, nullptr) == RP_EINVAL ||
               info.num_items == 0,
           "rp_run must refuse a NaN scale", iter);

    // FP8 K/V (one byte per element)
    Buf k8((size_t)b.rows_kv * b.hkv * b.d), v8((size_t)b.rows_kv * b.hkv * b.d);
    st = rp_run_fp8kv(plan, q.p, k8.p, v8.p, 0.5f, 2.0f, o.p, (float *)lse.p, scale, wsb ? ws.p : nullptr,
                      wsb, nullptr);
    expect(st == RP_OK, "rp_run_fp8kv", iter);

    // paged K/V: pages in random order, padded table
    static const int page_sizes[] = {16, 32, 64, 128};
    const int ps = page_sizes[rnd() % 4];
    int max_blocks = 1, pages = 0;
    for (int r = 0; r < b.batch; ++r) {
        const int need = (b.ki[r + 1] - b.ki[r] + ps - 1) / ps;
        max_blocks = need > max_blocks ? need : max_blocks;
        pages += need;
    }
    max_blocks += (int)(rnd() % 3);
    const int pool = pages + 2;
    std::vector<int32_t> table((size_t)(b.batch ? b.batch : 1) * max_blocks);
    int next = 0;
    for (int r = 0; r < b.batch; ++r) {
        const int need = (b.ki[r + 1] - b.ki[r] + ps - 1) / ps;
        for (int c = 0; c < max_blocks; ++c) {
            const int kind = (int)(rnd() % 3);
            table[(size_t)r * max_blocks + c] =
                c < need ? (next++ * 7919) % pool : (kind == 0 ? -1 : kind == 1 ? 0 : (int)(rnd() % pool));
        }
    }
    const size_t pool_b = (size_t)pool * ps * b.hkv * b.d * 2;
    Buf kp(pool_b), vp(pool_b), tab(table.size() * 4);
    std::memcpy(tab.p, table.data(), table.size() * 4);
    st = rp_run_paged(plan, q.p, kp.p, vp.p, (const int32_t *)tab.p, max_blocks, ps, o.p, (float *)lse.p,
                      scale, wsb ? ws.p : nullptr, wsb, nullptr);
    expect(st == RP_OK, "rp_run_paged", iter);
    if (max_blocks > 1 && info.num_items > 0) {
        int64_t longest = 0;
        for (int r = 0; r < b.batch; ++r)
            longest = b.ki[r + 1] - b.ki[r] > longest ? b.ki[r + 1] - b.ki[r] : longest;
        if ((longest + ps - 1) / ps > 1)
            expect(rp_run_paged(plan, q.p, kp.p, vp.p, (const int32_t *)tab.p, (int)((longest + ps - 1) / ps) - 1,
                                ps, o.p, (float *)lse.p, scale, ws.p, wsb, nullptr) == RP_EINVAL,
                   "rp_run_paged must refuse a short table", iter);
    }
    rp_plan_destroy(plan);

    // one-shot entry point on one of 11 stream handles (more than the
    // per-device cache holds), so plans and workspaces are evicted
    void *stream = (void *)(uintptr_t)(1 + iter % 11);
    st = ragged_prefill_bf16(q.p, k.p, v.p, o.p, (float *)lse.p, b.qi.data(), b.ki.data(), b.batch, b.hq,
                             b.hkv, b.d, b.causal, scale, stream);
    expect(st == RP_OK, "ragged_prefill_bf16", iter);

    // shared prefix over the same batch (causal needs qo <= kv everywhere)
    bool qo_le_kv = true;
    for (int r = 0; r < b.batch; ++r)
        qo_le_kv = qo_le_kv && b.qi[r + 1] - b.qi[r] <= b.ki[r + 1] - b.ki[r];
    const int shared_len = (int)(rnd() % 300);
    rp_plan *sp = nullptr;
    st = rp_plan_create_shared_prefix(b.qi.data(), b.ki.data(), b.batch, shared_len, b.hq, b.hkv, b.d,
                                      b.causal, &opts, &sp);
    if (b.causal && !qo_le_kv && shared_len > 0) {
        expect(st == RP_EINVAL, "shared prefix must refuse qo > kv under causal", iter);
    } else {
        expect(st == RP_OK, "rp_plan_create_shared_prefix", iter);
        if (st == RP_OK) {
            const size_t swb = rp_plan_workspace_bytes(sp);
            Buf sws(swb), ks((size_t)shared_len * b.hkv * b.d * 2), vs((size_t)shared_len * b.hkv * b.d * 2);
            st = rp_run_shared_prefix(sp, q.p, ks.p, vs.p, k.p, v.p, o.p, (float *)lse.p, scale, sws.p, swb,
                                      nullptr);
            expect(st == RP_OK, "rp_run_shared_prefix", iter);
            rp_plan_destroy(sp);
        }
    }
}

void invalid_inputs(int iter)
{
    const int32_t qi[] = {0, 5, 3}, ki[] = {0, 5, 9}, ok[] = {0, 5, 9};
    rp_plan *p = nullptr;
    expect(rp_plan_create(qi, ki, 2, 8, 2, 128, 1, nullptr, &p) == RP_EINVAL && !p, "decreasing q offsets", iter);
    const int32_t neg[] = {-2, 5, 9};
    expect(rp_plan_create(neg, ok, 2, 8, 2, 128, 1, nullptr, &p) == RP_EINVAL, "negative offset", iter);
    expect(rp_plan_create(nullptr, ok, 2, 8, 2, 128, 1, nullptr, &p) == RP_EINVAL, "null offsets", iter);
    expect(rp_plan_create(ok, ok, 2, 8, 3, 128, 1, nullptr, &p) == RP_EINVAL, "heads not a multiple", iter);
    expect(rp_plan_create(ok, ok, 2, 8, 2, 96, 1, nullptr, &p) == RP_EUNSUPPORTED, "head_dim 96", iter);
    rp_plan_opts o{};
    o.split_mode = 3;
    expect(rp_plan_create(ok, ok, 2, 8, 2, 128, 1, &o, &p) == RP_EINVAL, "split mode 3", iter);
    o.split_mode = 0;
    o.kv_chunk = 100;
    expect(rp_plan_create(ok, ok, 2, 8, 2, 128, 1, &o, &p) == RP_EINVAL, "kv_chunk 100", iter);
    expect(rp_merge_state(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 4, 8, 128, nullptr) == RP_EINVAL,
           "merge with null states", iter);
    expect(rp_merge_states(nullptr, nullptr, nullptr, nullptr, 4, 0, 8, 128, nullptr) == RP_EINVAL,
           "merge of zero states", iter);
    expect(rp_run(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1.0f, nullptr, 0, nullptr) == RP_EINVAL,
           "run without a plan", iter);
}

void merges(int iter)
{
    const int rows = (int)(rnd() % 40), heads = 1 + (int)(rnd() % 9), d = 8 << (rnd() % 7);
    const int k = 1 + (int)(rnd() % 5);
    Buf va((size_t)rows * heads * d * 2), vb((size_t)rows * heads * d * 2), out((size_t)rows * heads * d * 2);
    Buf sa((size_t)rows * heads * 4), sb((size_t)rows * heads * 4), so((size_t)rows * heads * 4);
    expect(rp_merge_state(va.p, (float *)sa.p, vb.p, (float *)sb.p, out.p, (float *)so.p, rows, heads, d,
                          nullptr) == RP_OK, "rp_merge_state", iter);
    expect(rp_merge_state_in_place(va.p, (float *)sa.p, vb.p, (float *)sb.p, rows, heads, d, nullptr) == RP_OK,
           "rp_merge_state_in_place", iter);
    Buf vk((size_t)rows * k * heads * d * 2), sk((size_t)rows * k * heads * 4);
    expect(rp_merge_states(vk.p, (float *)sk.p, out.p, nullptr, rows, k, heads, d, nullptr) == RP_OK,
           "rp_merge_states", iter);
}

void injected_alloc_failure(int iter)
{
    // a batch that needs a workspace (decode-like request, 2048-key chunks)
    const int32_t qi[] = {0, 1, 41}, ki[] = {0, 5000 + iter, 5100 + iter};
    const size_t qb = 41 * 8 * 128 * 2, kb = (size_t)(5100 + iter) * 2 * 128 * 2;
    Buf q(qb), k(kb), v(kb), o(qb, 0xab), lse(41 * 8 * 4, 0xcd);
    setenv("RP_FAULT_INJECT", "alloc", 1);
    rp_plan *p = nullptr;
    expect(rp_plan_create(qi, ki, 2, 8, 2, 128, 1, nullptr, &p) == RP_ENOMEM && p == nullptr,
           "rp_plan_create under injected allocation failure", iter);
    const int st = ragged_prefill_bf16(q.p, k.p, v.p, o.p, (float *)lse.p, qi, ki, 2, 8, 2, 128, 1, 0.088f,
                                       (void *)(uintptr_t)(100 + iter));
    expect(st == RP_ENOMEM, "one-shot call under injected allocation failure", iter);
    bool untouched = true;
    for (size_t i = 0; i < qb; ++i)
        untouched = untouched && static_cast<unsigned char *>(o.p)[i] == 0xab;
    for (size_t i = 0; i < 41 * 8 * 4; ++i)
        untouched = untouched && static_cast<unsigned char *>(lse.p)[i] == 0xcd;
    expect(untouched, "outputs must stay untouched after RP_ENOMEM", iter);
    unsetenv("RP_FAULT_INJECT");
    expect(ragged_prefill_bf16(q.p, k.p, v.p, o.p, (float *)lse.p, qi, ki, 2, 8, 2, 128, 1, 0.088f,
                               (void *)(uintptr_t)(100 + iter)) == RP_OK,
           "one-shot call after the injection ends", iter);
}

}  // namespace

int main(int argc, char **argv)
{
    const int iters = argc > 1 ? std::atoi(argv[1]) : 200;
    for (int it = 0; it < iters; ++it) {
        Batch b = random_batch();
        run_batch(b, it);
        merges(it);
        if (it % 10 == 0) {
            invalid_inputs(it);
            injected_alloc_failure(it);
        }
    }
    if (fails) {
        std::fprintf(stderr, "abi driver: %d failures\n", fails);
        return 1;
    }
    std::printf("abi driver: ok (%d batches)\n", iters);
    return 0;
}
