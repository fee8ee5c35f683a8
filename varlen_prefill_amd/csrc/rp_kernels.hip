// gfx950 (CDNA4) kernels of the ragged prefill attention library.
//
// tile_kernel: one workgroup (4 waves) per tile work item.  The tile holds up
// to 128 rows = (query token, qo head) pairs of one request and one GQA group;
// each wave owns 32 rows.  For every key block of the item's key range the
// workgroup stages K and V from HBM into double-buffered LDS (16-byte
// coalesced loads), and each wave computes
//   S^T = K Q^T          bf16 MFMA 32x32x16, fp32 accumulation
//   online softmax       row max / sum held in registers; the two lanes that
//                        share a row combine with one permlane32 swap
//   O^T += V^T P^T       bf16 MFMA; V read with the LDS transpose read
// (the tiled online-softmax computation of FlashAttention-2, page "Module
// flashinfer", module doc, re-designed for 64-wide waves and MFMA).  Working
// with transposed products keeps every row's scores inside one lane pair and
// lets P feed the second MFMA straight from registers.
//
// P is rounded to bf16 for the PV MFMA.  On key blocks that are partially
// masked for the tile, and on every block of tiles whose first row sees at
// most kHiLoKeys keys, P is split into bf16 hi + bf16 lo (two MFMAs), which
// keeps rows with few keys accurate to well under one bf16 ulp of O.
//
// merge_kernel: folds the fp32 partial states of split tiles, chunk by chunk
// in ascending key order (merge of attention states, page
// "flashinfer-ai/flashinfer", "Merge Attention States"), and writes bf16 O
// and the natural-log LSE.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "rp_internal.h"

namespace rp {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLn2 = 0.693147180559945309f;

template <int HD>
struct Tile {
    static constexpr int BK = key_block(HD);     // keys per block
    static constexpr int NB = BK / 32;           // 32-key MFMA row blocks of S^T
    static constexpr int DS = HD / 16;           // k-steps of the QK^T MFMA
    static constexpr int DB = HD / 32;           // 32-wide d blocks of O^T
    static constexpr int KST = HD + 8;           // LDS row stride of K (bf16): 8-row phases hit distinct banks
    static constexpr int VST = HD + 16;          // LDS row stride of V (bf16): 4-row transpose reads hit distinct banks
    static constexpr int KTILE = BK * KST;
    static constexpr int VTILE = BK * VST;
    static constexpr int CPR = HD / 8;           // 16-byte chunks per K/V row
    static constexpr int NLOAD = BK * CPR / kThreads;
    static constexpr int LDS_BYTES = 2 * (KTILE + VTILE) * 2;
    static_assert(NLOAD * kThreads == BK * CPR, "block must split evenly over threads");
};

__device__ inline float pair_max(float x)
{
    // lanes l and l^32 hold the two halves of one row's keys
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                              __builtin_bit_cast(unsigned, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ inline float pair_sum(float x)
{
    // r[0] is the lower lane's value, r[1] the upper lane's, in both lanes:
    // both lanes add in the same order and get the same bits
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                              __builtin_bit_cast(unsigned, x), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Fold state b into state a (base-2 log-sum-exp, normalised outputs):
//   lse = log2(2^lse_a + 2^lse_b),  o = o_a 2^(lse_a - lse) + o_b 2^(lse_b - lse).
// Written without fma contraction so that every caller rounds identically.
template <int N>
__device__ inline void fold_state(float &lse_a, float (&o_a)[N], float lse_b, const float (&o_b)[N])
{
#pragma clang fp contract(off)
    const float mx = fmaxf(lse_a, lse_b);
    if (mx == -INFINITY)
        return;
    const float wa = fast_exp2(lse_a - mx);
    const float wb = fast_exp2(lse_b - mx);
    const float s = wa + wb;
    const float inv = 1.0f / s;
    const float ca = wa * inv;
    const float cb = wb * inv;
#pragma unroll
    for (int i = 0; i < N; ++i)
        o_a[i] = o_a[i] * ca + o_b[i] * cb;
    lse_a = mx + log2f(s);
}

template <int HD, bool POS_SCALE>
__device__ inline void tile_body(const TileArgs &a, const Item &it, __bf16 *smem)
{
    using T = Tile<HD>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int h = lane >> 5;          // which half of the wave
    const int qc = lane & 31;         // MFMA column = the wave's row
    const int g = a.group;
    const int r = w * 32 + qc;        // tile row
    const int tok = r / g;
    const int hig = r - tok * g;
    const bool row_valid = tok < it.n_tok;
    const int head = it.kv_head * g + hig;
    const int t_row = it.t0 + tok;
    const size_t q_row = (size_t)(it.q_tok0 + (row_valid ? tok : 0)) * a.num_qo_heads + head;

    int lim_row = it.kv_len;
    if (a.causal) {
        int lr = t_row + it.kv_len - it.qo_len + 1;
        lim_row = lr < 0 ? 0 : (lr > it.kv_len ? it.kv_len : lr);
    }

    // Q fragments: B operand of S^T = K Q^T; lane holds Q[row][16 ds + 8 h .. +7]
    bf16x8 qf[T::DS];
    {
        const bf16x8 *qp = reinterpret_cast<const bf16x8 *>(
            static_cast<const __bf16 *>(a.q) + q_row * HD + 8 * h);
#pragma unroll
        for (int ds = 0; ds < T::DS; ++ds) {
            if (row_valid) {
                qf[ds] = qp[2 * ds];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    qf[ds][e] = (__bf16)0.0f;
            }
        }
    }

    f32x16 acc[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            acc[db][j] = 0.0f;
    float m = -INFINITY;   // running max of scaled scores (log2 units)
    float l = 0.0f;        // this lane's part of the running sum

    const float c = a.scale_log2;
    const int kb_begin = it.key_begin / T::BK;
    const int kb_end = it.key_end > it.key_begin ? (it.key_end + T::BK - 1) / T::BK : kb_begin;
    const bool hilo_all = it.lim_first <= kHiLoKeys;

    const size_t kv_stride = (size_t)a.num_kv_heads * HD;
    const __bf16 *kbase = static_cast<const __bf16 *>(a.k) +
                          ((size_t)it.kv_row0 * a.num_kv_heads + it.kv_head) * HD;
    const __bf16 *vbase = static_cast<const __bf16 *>(a.v) +
                          ((size_t)it.kv_row0 * a.num_kv_heads + it.kv_head) * HD;

    uint4 kst[T::NLOAD], vst[T::NLOAD];
    auto gload = [&](int kb) {
#pragma unroll
        for (int i = 0; i < T::NLOAD; ++i) {
            const int ci = tid + i * kThreads;
            const int key = ci / T::CPR;
            const int cc = ci - key * T::CPR;
            const int kk = kb * T::BK + key;
            if (kk < it.kv_len) {
                kst[i] = *reinterpret_cast<const uint4 *>(kbase + (size_t)kk * kv_stride + 8 * cc);
                vst[i] = *reinterpret_cast<const uint4 *>(vbase + (size_t)kk * kv_stride + 8 * cc);
            } else {
                kst[i] = make_uint4(0, 0, 0, 0);
                vst[i] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto lstore = [&](int buf) {
        __bf16 *Ks = smem + buf * (T::KTILE + T::VTILE);
        __bf16 *Vs = Ks + T::KTILE;
#pragma unroll
        for (int i = 0; i < T::NLOAD; ++i) {
            const int ci = tid + i * kThreads;
            const int key = ci / T::CPR;
            const int cc = ci - key * T::CPR;
            *reinterpret_cast<uint4 *>(Ks + key * T::KST + 8 * cc) = kst[i];
            *reinterpret_cast<uint4 *>(Vs + key * T::VST + 8 * cc) = vst[i];
        }
    };

    if (kb_begin < kb_end) {
        gload(kb_begin);
        lstore(0);
    }
    __syncthreads();

    const int grp = lane >> 4;
    const int s16 = lane & 15;

    for (int kb = kb_begin; kb < kb_end; ++kb) {
        const int buf = (kb - kb_begin) & 1;
        const bool more = kb + 1 < kb_end;
        if (more)
            gload(kb + 1);

        const __bf16 *Ks = smem + buf * (T::KTILE + T::VTILE);
        const __bf16 *Vs = Ks + T::KTILE;

        // ---- S^T = K Q^T ----
        f32x16 s[T::NB];
#pragma unroll
        for (int n = 0; n < T::NB; ++n)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                s[n][j] = 0.0f;
#pragma unroll
        for (int ds = 0; ds < T::DS; ++ds) {
#pragma unroll
            for (int n = 0; n < T::NB; ++n) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(
                    Ks + (32 * n + qc) * T::KST + 16 * ds + 8 * h);
                s[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], s[n], 0, 0, 0);
            }
        }

        // ---- mask + online softmax ----
        const int key0 = kb * T::BK;
        const bool need_mask = key0 + T::BK > it.lim_first;
        const bool hilo = hilo_all || need_mask;
        float p[T::NB][16];
        float mx = -INFINITY;
        if (POS_SCALE) {
            if (need_mask) {
#pragma unroll
                for (int n = 0; n < T::NB; ++n)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = key0 + 32 * n + 8 * (j >> 2) + 4 * h + (j & 3);
                        if (key >= lim_row)
                            s[n][j] = -INFINITY;
                    }
            }
#pragma unroll
            for (int n = 0; n < T::NB; ++n)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    mx = fmaxf(mx, s[n][j]);
            mx = pair_max(mx) * c;
        } else {
#pragma unroll
            for (int n = 0; n < T::NB; ++n)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    float x = s[n][j] * c;
                    if (need_mask) {
                        const int key = key0 + 32 * n + 8 * (j >> 2) + 4 * h + (j & 3);
                        if (key >= lim_row)
                            x = -INFINITY;
                    }
                    s[n][j] = x;
                    mx = fmaxf(mx, x);
                }
            mx = pair_max(mx);
        }
        const float m_new = fmaxf(m, mx);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m - m_use);
        float psum = 0.0f;
#pragma unroll
        for (int n = 0; n < T::NB; ++n)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float x = POS_SCALE ? __builtin_fmaf(s[n][j], c, -m_use) : s[n][j] - m_use;
                p[n][j] = fast_exp2(x);
                psum += p[n][j];
            }
        l = l * alpha + psum;
        m = m_new;
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    acc[db][j] *= alpha;
        }

        // ---- P to bf16 (B operand of O^T += V^T P^T) ----
        // MFMA k-step t of key row block n: lane half h, element e holds key
        // 32 n + 16 t + 4 h + 8 (e / 4) + e % 4 — the keys this lane already
        // holds in S^T registers j = 8 t + e.
        bf16x8 ph[T::NB][2], pl[T::NB][2];
#pragma unroll
        for (int n = 0; n < T::NB; ++n)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pv = p[n][8 * t + e];
                    const __bf16 hb = (__bf16)pv;
                    ph[n][t][e] = hb;
                    pl[n][t][e] = (__bf16)(pv - (float)hb);
                }

        // ---- O^T += V^T P^T ----
        // A operand: lane (h, d = 32 db + lane % 32) needs V[key][d] for the
        // 8 keys above; two LDS transpose reads each deliver 4 consecutive keys.
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
#pragma unroll
            for (int n = 0; n < T::NB; ++n) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const __bf16 *vp = Vs + (32 * n + 16 * t + 4 * h + (s16 >> 2)) * T::VST +
                                       32 * db + 16 * (grp & 1) + 4 * (s16 & 3);
                    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) __bf16 *)vp));
                    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)((__attribute__((address_space(3))) __bf16 *)(vp + 8 * T::VST)));
                    // join the two 4-key halves as one 16-byte vector (element-wise
                    // inserts into a bf16 vector are not lowered reliably)
                    const i16x8 v01 = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, v01);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, ph[n][t], acc[db], 0, 0, 0);
                    if (hilo)
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[n][t], acc[db], 0, 0, 0);
                }
            }
        }

        if (more)
            lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
    const float lt = pair_sum(l);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const float lse2 = lt > 0.0f ? m + log2f(lt) : -INFINITY;
    if (!row_valid)
        return;
    if (it.slot < 0) {
        __bf16 *op = static_cast<__bf16 *>(a.o) + q_row * HD + 4 * h;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ov[e] = (__bf16)(acc[db][4 * jj + e] * inv);
                *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * jj) = ov;
            }
        if (h == 0 && a.lse != nullptr)
            a.lse[q_row] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
    } else {
        float *pp = a.part_o + ((size_t)it.slot * kTileRows + r) * HD + 4 * h;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float4 ov;
                ov.x = acc[db][4 * jj + 0] * inv;
                ov.y = acc[db][4 * jj + 1] * inv;
                ov.z = acc[db][4 * jj + 2] * inv;
                ov.w = acc[db][4 * jj + 3] * inv;
                *reinterpret_cast<float4 *>(pp + 32 * db + 8 * jj) = ov;
            }
        if (h == 0)
            a.part_lse[(size_t)it.slot * kTileRows + r] = lse2;
    }
}

template <int HD>
__global__ __launch_bounds__(kThreads, HD == 128 ? 2 : 1) void tile_kernel(TileArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    __bf16 *smem = reinterpret_cast<__bf16 *>(smem_raw);
    const Item it = a.items[blockIdx.x];
    if (a.scale_log2 > 0.0f)
        tile_body<HD, true>(a, it, smem);
    else
        tile_body<HD, false>(a, it, smem);
}

template <int HD>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a)
{
    const MergeItem it = a.items[blockIdx.x];
    const int rows = it.n_tok * a.group;
    constexpr int CPR = HD / 8;
    for (int task = threadIdx.x; task < rows * CPR; task += kMergeThreads) {
        const int r = task / CPR;
        const int cc = task - r * CPR;
        float lse_run = a.part_lse[(size_t)it.slot0 * kTileRows + r];
        float o_run[8];
        {
            const float4 *src = reinterpret_cast<const float4 *>(
                a.part_o + ((size_t)it.slot0 * kTileRows + r) * HD + 8 * cc);
            const float4 x0 = src[0], x1 = src[1];
            o_run[0] = x0.x; o_run[1] = x0.y; o_run[2] = x0.z; o_run[3] = x0.w;
            o_run[4] = x1.x; o_run[5] = x1.y; o_run[6] = x1.z; o_run[7] = x1.w;
        }
        for (int ch = 1; ch < it.n_chunks; ++ch) {
            const size_t slot = (size_t)it.slot0 + ch;
            const float lse_c = a.part_lse[slot * kTileRows + r];
            const float4 *src = reinterpret_cast<const float4 *>(a.part_o + (slot * kTileRows + r) * HD + 8 * cc);
            const float4 x0 = src[0], x1 = src[1];
            const float o_c[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            fold_state<8>(lse_run, o_run, lse_c, o_c);
        }
        const int tok = r / a.group;
        const int head = it.kv_head * a.group + (r - tok * a.group);
        const size_t q_row = (size_t)(it.q_tok0 + tok) * a.num_qo_heads + head;
        bf16x8 ov;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            ov[e] = (__bf16)o_run[e];
        *reinterpret_cast<bf16x8 *>(static_cast<__bf16 *>(a.o) + q_row * HD + 8 * cc) = ov;
        if (cc == 0 && a.lse != nullptr)
            a.lse[q_row] = lse_run == -INFINITY ? -INFINITY : lse_run * kLn2;
    }
}

template <int HD>
int launch_tile(const TileArgs &args, int64_t num_items, hipStream_t stream)
{
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&tile_kernel<HD>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           Tile<HD>::LDS_BYTES);
        if (e != hipSuccess)
            return (int)e;
        attr_set = true;
    }
    hipLaunchKernelGGL(tile_kernel<HD>, dim3((unsigned)num_items), dim3(kThreads),
                       Tile<HD>::LDS_BYTES, stream, args);
    return (int)hipGetLastError();
}

}  // namespace

int launch_tile_kernel(int head_dim, const TileArgs &args, int64_t num_items, void *stream)
{
    if (num_items <= 0)
        return (int)hipSuccess;
    if (num_items > INT_MAX)
        return (int)hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (head_dim == 128)
        return launch_tile<128>(args, num_items, s);
    if (head_dim == 256)
        return launch_tile<256>(args, num_items, s);
    return (int)hipErrorInvalidValue;
}

int launch_merge_kernel(int head_dim, const MergeArgs &args, int64_t num_items, void *stream)
{
    if (num_items <= 0)
        return (int)hipSuccess;
    if (num_items > INT_MAX)
        return (int)hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (head_dim == 128)
        hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)num_items), dim3(kMergeThreads), 0, s, args);
    else if (head_dim == 256)
        hipLaunchKernelGGL(merge_kernel<256>, dim3((unsigned)num_items), dim3(kMergeThreads), 0, s, args);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // namespace rp
