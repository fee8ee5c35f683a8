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
// P enters the PV MFMA either rounded to bf16 or split into bf16 hi + bf16
// lo parts (two MFMAs, accurate to about 2^-17), which keeps output elements
// within the error gate where single keys carry much of a row's softmax:
//  * tiles whose rows see few keys split P on every block;
//  * other final items round P, and a workgroup whose result holds an
//    element with |O| >= kRecomputeAbsO (where the output's own bf16
//    rounding leaves little of the gate) computes the item again with P
//    split on every block;
//  * partial states of split-KV tiles (merged later, so not recomputable)
//    split P in the key blocks where some row of the wave has a key whose p
//    exceeds kHiLoFracPartial of the row's running sum.
// Every decision reads only the tile's own scores and outputs, so results
// stay independent of the batch.
//
// merge_kernel: folds the fp32 partial states of split tiles, chunk by chunk
// in ascending key order (merge of attention states, page
// "flashinfer-ai/flashinfer", "Merge Attention States"), and writes bf16 O
// and the natural-log LSE.
//
// Fold items (in-workgroup chunk folding): one workgroup runs all canonical
// KV chunks of a tile in order, each from a fresh state by the rules of a
// split item, and folds each chunk's normalised state into a running state
// in its workspace slot with the merge kernel's arithmetic and order, then
// writes O and LSE itself: the same bits as split items + merge kernel,
// without the merge launch and with one partial-state slot per tile instead
// of one per chunk.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdint>
#include <type_traits>

#include "rp_internal.h"

// Built twice: RP_TILE_FOLD 0 gives the plain tile kernels, the merge kernel
// and the launchers; RP_TILE_FOLD 1 the tile kernels that also run fold
// items (in-workgroup chunk folding) and their launcher.
#ifndef RP_TILE_FOLD
#define RP_TILE_FOLD 0
#endif

namespace rp {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLn2 = 0.693147180559945309f;
// lazy-rescale threshold in log2 units
constexpr float kRescaleLog2 = 8.0f;
// a lane's part of a block's row sum at most this (2^(threshold - 1)) keeps
// the reference max (fast path of the softmax update)
constexpr float kFastSumMax = 128.0f;

// Wave layout.  head_dim 128: 4 waves of 32 rows (32x32x16 MFMAs), two
// workgroups per CU.  head_dim 256: 8 waves of 16 rows (16x16x32 MFMAs), one
// workgroup per CU.  Both run two waves per SIMD, so that one wave's softmax
// and LDS latency overlap the other's MFMAs; at head_dim 256 32-row waves
// would need about twice the registers and leave one wave per SIMD.
template <int HD>
struct Tile {
    static constexpr int RPW = HD == 128 ? 32 : 16;   // tile rows per wave
    static constexpr int NW = kTileRows / RPW;         // waves per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int BK = key_block(HD);     // keys per block
    static constexpr int NB = BK / 32;           // 32-key MFMA row blocks of S^T (32-row waves)
    static constexpr int DS = HD / 16;           // k-steps of the QK^T MFMA (32-row waves)
    static constexpr int DB = HD / 32;           // 32-wide d blocks of O^T (32-row waves)
    static constexpr int KS16 = HD / 32;         // k-steps of the QK^T MFMA (16-row waves)
    static constexpr int DT16 = HD / 16;         // 16-wide d tiles of O^T (16-row waves)
    static constexpr int RB = HD * 2;            // bytes per K/V row in LDS (unpadded)
    static constexpr int CPR = HD / 8;           // 16-byte chunks per row
    static constexpr int TILE_BYTES = BK * RB;   // one K (or V) block
    static constexpr int STAGE_BYTES = 2 * TILE_BYTES;     // K and V of one block
    static constexpr int STAGES = kv_stages(HD);           // blocks in flight
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    // direct-to-LDS loads: one instruction moves 64 lanes x 16 bytes
    static constexpr int NLOAD = TILE_BYTES / (64 * 16) / NW;
    static_assert(NLOAD * 64 * 16 * NW == TILE_BYTES, "block must split evenly over waves");
    static_assert(RPW == 32 || BK == 32, "16-row waves take a 32-key block as one PV k-step");
};

// LDS layout: chunk c (16 bytes) of key row r sits at chunk position
// c ^ swz(r) of that row (rows are 256 or 512 bytes, a multiple of the 64
// four-byte banks).  K is read 16 rows at a time at one chunk (128-bit reads
// are served 16 lanes per cycle): swizzle r & 15 puts those rows on distinct
// 16-byte slots.  V is read by the transpose read, 32 lanes per cycle: with
// 32-row waves (head_dim 128) over 4 rows x 4 adjacent chunks, where swizzle
// 4 (r & 3) moves each row to its own 4-chunk group; with 16-row waves
// (head_dim 256) over 8 rows x 2 adjacent chunks, where swizzle 2 (r & 7)
// moves each row to its own chunk pair.
__device__ inline int swz_k(int r) { return r & 15; }
template <int HD>
__device__ inline int swz_v(int r) { return HD == 128 ? (r & 3) << 2 : (r & 7) << 1; }

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

// 16-row waves: lanes l, l^16, l^32, l^48 hold the four parts of one row's
// keys.  Every lane computes (x0 op x1) op (x2 op x3) and gets the same bits.
__device__ inline float quad_max(float x)
{
    auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                              __builtin_bit_cast(unsigned, x), false, false);
    const float y = fmaxf(__builtin_bit_cast(float, (unsigned)a[0]), __builtin_bit_cast(float, (unsigned)a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, y),
                                              __builtin_bit_cast(unsigned, y), false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)b[0]), __builtin_bit_cast(float, (unsigned)b[1]));
}

__device__ inline float quad_sum(float x)
{
    auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                              __builtin_bit_cast(unsigned, x), false, false);
    const float y = __builtin_bit_cast(float, (unsigned)a[0]) + __builtin_bit_cast(float, (unsigned)a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, y),
                                              __builtin_bit_cast(unsigned, y), false, false);
    return __builtin_bit_cast(float, (unsigned)b[0]) + __builtin_bit_cast(float, (unsigned)b[1]);
}

// the row sum of the lanes' parts, in the wave layout of head_dim HD
template <int HD>
__device__ inline float row_sum(float x) { return Tile<HD>::RPW == 32 ? pair_sum(x) : quad_sum(x); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Fold of state b into state a (base-2 log-sum-exp, normalised outputs):
//   lse = log2(2^lse_a + 2^lse_b),  o = o_a 2^(lse_a - lse) + o_b 2^(lse_b - lse).
// Written without fma contraction so that every caller (the merge kernel and
// the tile kernel's in-workgroup fold) rounds identically.  keep: both states
// are empty (lse -inf), a stays as it is.
struct FoldWeights {
    float ca, cb, lse;
    bool keep;
};

__device__ inline FoldWeights fold_weights(float lse_a, float lse_b)
{
#pragma clang fp contract(off)
    FoldWeights f;
    const float mx = fmaxf(lse_a, lse_b);
    f.keep = mx == -INFINITY;
    const float wa = fast_exp2(lse_a - mx);
    const float wb = fast_exp2(lse_b - mx);
    const float s = wa + wb;
    const float inv = 1.0f / s;
    f.ca = wa * inv;
    f.cb = wb * inv;
    f.lse = f.keep ? lse_a : mx + log2f(s);
    return f;
}

__device__ inline float fold_value(const FoldWeights &f, float o_a, float o_b)
{
#pragma clang fp contract(off)
    return f.keep ? o_a : o_a * f.ca + o_b * f.cb;
}

// Registers one wave carries through a tile.
template <int HD, bool R16 = (Tile<HD>::RPW == 16)>
struct WaveState {
    bf16x8 qf[Tile<HD>::DS];   // Q fragments (B operand of S^T = K Q^T)
    f32x16 acc[Tile<HD>::DB];  // O^T accumulators
    float m;                   // running max of scaled scores (log2 units)
    float l;                   // this lane's part of the running sum
};

// 16-row waves
template <int HD>
struct WaveState<HD, true> {
    bf16x8 qf[Tile<HD>::KS16];  // Q fragments, 32 d per k-step
    f32x4 acc[Tile<HD>::DT16];  // O^T accumulators, 16 d per tile
    float m;
    float l;
};

// One key block of one wave: S^T = K Q^T, mask, online softmax update,
// O^T += V^T P^T.  MASK: the block holds keys beyond some row's causal limit
// (the diagonal or the KV tail); thr is this lane's visible-key bound
// relative to the block start and lane half; valid: this lane's row is a
// row of the tile.  FORCE and trig choose how P enters the PV product (see
// below).  Each variant is straight-line code so that LDS reads, MFMAs and
// VALU work can be interleaved.
template <int HD, bool POS_SCALE, bool MASK, bool FORCE>
__device__ __attribute__((always_inline)) inline void block_step(
    WaveState<HD> &st, const char *Ks, const char *Vs, float c, int thr, bool valid, bool trig,
    float kappa, int qc, int h, int grp, int s16)
{
    using T = Tile<HD>;
    f32x16 s[T::NB];
#pragma unroll
    for (int n = 0; n < T::NB; ++n)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            s[n][j] = 0.0f;
    // All K fragments of the block are requested up front; the MFMAs then
    // consume them in arrival order.
    bf16x8 kf[T::DS][T::NB];
#pragma unroll
    for (int ds = 0; ds < T::DS; ++ds)
#pragma unroll
        for (int n = 0; n < T::NB; ++n) {
            const int row = 32 * n + qc;
            kf[ds][n] = *reinterpret_cast<const bf16x8 *>(
                Ks + row * T::RB + 16 * ((2 * ds + h) ^ swz_k(row)));
        }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ds = 0; ds < T::DS; ++ds)
#pragma unroll
        for (int n = 0; n < T::NB; ++n)
            s[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds][n], st.qf[ds], s[n], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // The V fragments of the PV product are requested now and arrive while
    // the softmax runs.  A operand: lane (h, d = 32 db + lane % 32) needs
    // V[key][d] for the 8 keys of the P operand below; each LDS transpose
    // read delivers 4 consecutive keys.
    bf16x8 vf[T::DB][T::NB][2];
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
#pragma unroll
        for (int n = 0; n < T::NB; ++n) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                // source lane s16 of each 16-lane group reads key row
                // 32 n + 16 t + 4 h + s16 / 4 (and 8 rows further), d = 32 db +
                // 16 (grp & 1) + 4 (s16 & 3): chunk c, byte 8 (s16 & 1) within it
                const int row = 32 * n + 16 * t + 4 * h + (s16 >> 2);
                const int cc = 4 * db + 2 * (grp & 1) + ((s16 & 3) >> 1);
                const char *vp = Vs + row * T::RB + 16 * (cc ^ swz_v<HD>(row)) + 8 * (s16 & 1);
                const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)((__attribute__((address_space(3))) char *)vp));
                const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)((__attribute__((address_space(3))) char *)(vp + 8 * T::RB)));
                // join the two 4-key halves as one 16-byte vector (element-wise
                // inserts into a bf16 vector are not lowered reliably)
                const i16x8 v01 = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                vf[db][n][t] = __builtin_bit_cast(bf16x8, v01);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // S^T register j of row block n holds key 32 n + 8 (j / 4) + 4 h + j % 4
    float p[T::NB][16];
    float t8[T::NB * 8];
    // p = 2^(scaled score - m_use), and this lane's part of the row sum from
    // the fp32 P (the LSE needs it exact) as a fixed pairwise tree
    auto exp_sum = [&](float m_use) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < T::NB; ++n)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float x = POS_SCALE ? __builtin_fmaf(s[n][j], c, -m_use) : s[n][j] - m_use;
                p[n][j] = fast_exp2(x);
            }
#pragma unroll
        for (int n = 0; n < T::NB; ++n)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                t8[n * 8 + j] = p[n][2 * j] + p[n][2 * j + 1];
#pragma unroll
        for (int w = T::NB * 4; w >= 1; w >>= 1)
#pragma unroll
            for (int j = 0; j < w; ++j)
                t8[j] = t8[2 * j] + t8[2 * j + 1];
    };
    // Lazy rescaling: the reference max only moves when the block max
    // exceeds it by more than 2^8 (p <= 256 stays exact enough in bf16 and
    // fp32); O, l and the LSE are all taken relative to the same reference,
    // so the result does not depend on when it moves.
    //
    // Fast path (positive scale): P is first computed against the current
    // reference.  If every lane's part of the row sum is at most 2^7, every
    // p is, so no score of the block exceeds the reference by 8 (with a
    // margin of one binade for rounding) and the reference stays: those P
    // are exactly the ones the full update computes, and the block max is
    // never needed.  A reference still at -inf (no visible key yet) gives
    // p = inf or NaN, which fails the test.  Otherwise the wave takes the
    // full update below.
    //
    // FORCE: P enters the PV product split into bf16 hi + lo parts on every
    // block.  Otherwise, with trig (partial states of split-KV tiles), it is
    // split in blocks where some valid row of the wave has a key with
    // p > kHiLoFracPartial * (the row's running sum, this block included),
    // and rounded to bf16 elsewhere; without trig it is rounded to bf16 (the
    // caller recomputes the item where that matters).  A lane whose block
    // sum t is at most the fraction of its own running sum l + t holds no
    // such p (its sum is part of its row's): the fast path tests
    // t <= kappa l in every valid lane next to its own test (kappa = frac /
    // (1 - frac), infinite without trig), and only waves that fail it look
    // at the block's largest p.  Both tests come from the same values, so
    // the second branch does not wait for the VALU.
    constexpr bool FAST = POS_SCALE;
    bool full = true;
    bool check = !FORCE && trig;
    if (FAST) {
        if (MASK) {
#pragma unroll
            for (int n = 0; n < T::NB; ++n)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (32 * n + 8 * (j >> 2) + (j & 3) >= thr)
                        s[n][j] = -INFINITY;
        }
        const float lim_t = valid ? kappa * st.l : INFINITY;
        exp_sum(st.m);
        full = __any(!(t8[0] <= kFastSumMax));
        if (!FORCE)
            check = __any(t8[0] > lim_t);
    }
    if (__builtin_expect(full, !FAST)) {
        float mx = -INFINITY;
        if (POS_SCALE) {
#pragma unroll
            for (int n = 0; n < T::NB; ++n)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (!FAST && MASK && 32 * n + 8 * (j >> 2) + (j & 3) >= thr)
                        s[n][j] = -INFINITY;
                    mx = fmaxf(mx, s[n][j]);
                }
            mx = pair_max(mx) * c;
        } else {
#pragma unroll
            for (int n = 0; n < T::NB; ++n)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    float x = s[n][j] * c;
                    if (MASK && 32 * n + 8 * (j >> 2) + (j & 3) >= thr)
                        x = -INFINITY;
                    s[n][j] = x;
                    mx = fmaxf(mx, x);
                }
            mx = pair_max(mx);
        }
        const bool grow = mx > st.m + kRescaleLog2;
        const float m_ref = grow ? mx : st.m;
        const float m_use = m_ref == -INFINITY ? 0.0f : m_ref;
        exp_sum(m_use);
        if (__any(grow)) {
            const float alpha = fast_exp2(st.m - m_use);   // 1 where the reference stays, 0 at the start
            st.l *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db) {
                if constexpr (HD == 256) {
                    // The accumulators live in AGPRs (the MFMAs read and
                    // write them there).  Multiplied in place through one
                    // VGPR at a time, so that the copies to and from VGPRs
                    // stay in this rarely taken branch instead of being
                    // hoisted to the top of every key-block iteration.
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        float t;
                        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(t) : "a"(st.acc[db][j]));
                        t *= alpha;
                        asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(st.acc[db][j]) : "v"(t));
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        st.acc[db][j] *= alpha;
                }
            }
        }
        st.m = m_ref;
        check = !FORCE && trig;
    }
    st.l += t8[0];
    bool split = FORCE;
    if (!FORCE && __builtin_expect(check, !FAST)) {
        float pm = 0.0f;
#pragma unroll
        for (int n = 0; n < T::NB; ++n)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                pm = fmaxf(pm, p[n][j]);
        split = __any(valid && pm > kHiLoFracPartial * pair_sum(st.l));
    }

    // P as the B operand of O^T += V^T P^T: k-step t of row block n takes,
    // in lane half h, element e = key 32 n + 16 t + 4 h + 8 (e / 4) + e % 4,
    // i.e. this lane's S^T registers j = 8 t + e.
    bf16x8 ph[T::NB][2];
#pragma unroll
    for (int n = 0; n < T::NB; ++n)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ph[n][t][e] = (__bf16)p[n][8 * t + e];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int n = 0; n < T::NB; ++n)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][n][t], ph[n][t], st.acc[db], 0, 0, 0);
    if (__builtin_expect(split, 0)) {
        // the lo parts bf16(p - bf16(p))
        bf16x8 pl[T::NB][2];
#pragma unroll
        for (int n = 0; n < T::NB; ++n)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pl[n][t][e] = (__bf16)(p[n][8 * t + e] - (float)ph[n][t][e]);
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int n = 0; n < T::NB; ++n)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][n][t], pl[n][t], st.acc[db], 0, 0, 0);
    }
}

// One key block of one 16-row wave (head_dim 256): the same steps as
// block_step with 16x16x32 MFMAs.  Lane (n16 = lane % 16, j = lane / 16)
// holds row n16 of the wave.
//   S^T = K Q^T: two 16-key tiles t; k-step ks covers d 32 ks .. 32 ks + 31,
//     lane part j holding d 32 ks + 8 j .. + 7 of its key (A) and row (B);
//     the result's register i of tile t is key 16 t + 4 j + i.
//   O^T += V^T P^T: one k-step over the 32 keys; lane part j holds, as its
//     8 k-values, keys 4 j + e and 16 + 4 j + e (e < 4): exactly its own
//     S^T registers, so P never leaves the lane; the A operand (V^T, d tile
//     dt: d = 16 dt + n16) takes the same keys with two transpose reads.
// thr: this lane's visible-key bound relative to the block start and 4 j.
template <int HD, bool POS_SCALE, bool MASK, bool FORCE>
__device__ __attribute__((always_inline)) inline void block_step16(
    WaveState<HD> &st, const char *Ks, const char *Vs, float c, int thr, bool valid, bool trig,
    float kappa, int n16, int j)
{
    using T = Tile<HD>;
    constexpr int KS = T::KS16;
    constexpr int DT = T::DT16;
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s[t][i] = 0.0f;
    bf16x8 kf[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = 16 * t + n16;
            kf[ks][t] = *reinterpret_cast<const bf16x8 *>(Ks + row * T::RB + 16 * ((4 * ks + j) ^ swz_k(row)));
        }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < 2; ++t)
            s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks][t], st.qf[ks], s[t], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // V fragments of the first half of the d tiles, requested now so that
    // they arrive during the softmax (the second half is requested after the
    // first half's PV MFMAs are issued).  In each 16-lane group, source lane
    // n16 reads key row 16 u + 4 j + n16 / 4 at d = 16 dt + 4 (n16 % 4): lane
    // n16 then receives V[16 u + 4 j + e][16 dt + n16] for e = 0..3.
    auto read_v = [&](int dt) __attribute__((always_inline)) {
        i16x4 v[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int row = 16 * u + 4 * j + (n16 >> 2);
            const int cc = 2 * dt + ((n16 & 3) >> 1);
            const char *vp = Vs + row * T::RB + 16 * (cc ^ swz_v<HD>(row)) + 8 * (n16 & 1);
            v[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)((__attribute__((address_space(3))) char *)vp));
        }
        const i16x8 v01 = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v01);
    };
    constexpr int DH = DT / 2;
    bf16x8 vf[DT];
#pragma unroll
    for (int dt = 0; dt < DH; ++dt)
        vf[dt] = read_v(dt);
    __builtin_amdgcn_sched_barrier(0);
    // p[4 t + i]: key 16 t + 4 j + i
    float p[8];
    float tsum;
    auto exp_sum = [&](float m_use) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = POS_SCALE ? __builtin_fmaf(s[t][i], c, -m_use) : s[t][i] - m_use;
                p[4 * t + i] = fast_exp2(x);
            }
        tsum = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    };
    // Lazy rescale, fast path and the split of P exactly as in block_step;
    // the row's parts sit in four lanes instead of two.
    constexpr bool FAST = POS_SCALE;
    bool full = true;
    bool check = !FORCE && trig;
    if (FAST) {
        if (MASK) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * t + i >= thr)
                        s[t][i] = -INFINITY;
        }
        const float lim_t = valid ? kappa * st.l : INFINITY;
        exp_sum(st.m);
        full = __any(!(tsum <= kFastSumMax));
        if (!FORCE)
            check = __any(tsum > lim_t);
    }
    if (__builtin_expect(full, !FAST)) {
        float mx = -INFINITY;
        if (POS_SCALE) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (!FAST && MASK && 16 * t + i >= thr)
                        s[t][i] = -INFINITY;
                    mx = fmaxf(mx, s[t][i]);
                }
            mx = quad_max(mx) * c;
        } else {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = s[t][i] * c;
                    if (MASK && 16 * t + i >= thr)
                        x = -INFINITY;
                    s[t][i] = x;
                    mx = fmaxf(mx, x);
                }
            mx = quad_max(mx);
        }
        const bool grow = mx > st.m + kRescaleLog2;
        const float m_ref = grow ? mx : st.m;
        const float m_use = m_ref == -INFINITY ? 0.0f : m_ref;
        exp_sum(m_use);
        if (__any(grow)) {
            const float alpha = fast_exp2(st.m - m_use);
            st.l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st.acc[dt][i] *= alpha;
        }
        st.m = m_ref;
        check = !FORCE && trig;
    }
    st.l += tsum;
    bool split = FORCE;
    if (!FORCE && __builtin_expect(check, !FAST)) {
        float pm = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            pm = fmaxf(pm, p[e]);
        split = __any(valid && pm > kHiLoFracPartial * quad_sum(st.l));
    }
    bf16x8 ph;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        ph[e] = (__bf16)p[e];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < DH; ++dt)
        st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], ph, st.acc[dt], 0, 0, 0);
#pragma unroll
    for (int dt = DH; dt < DT; ++dt)
        vf[dt] = read_v(dt);
#pragma unroll
    for (int dt = DH; dt < DT; ++dt)
        st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], ph, st.acc[dt], 0, 0, 0);
    if (__builtin_expect(split, 0)) {
        bf16x8 pl;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            pl[e] = (__bf16)(p[e] - (float)ph[e]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pl, st.acc[dt], 0, 0, 0);
    }
}

template <int HD, bool POS_SCALE, bool PAGED, bool FP8, bool FOLD>
__device__ inline void tile_body(const TileArgs &a, const Item &it, char *smem, int fc)
{
    using T = Tile<HD>;
    constexpr bool R16 = T::RPW == 16;
    int tid = threadIdx.x;
    // (the lane values of chunk fc are recomputed from an opaque thread id:
    // hoisted out of the chunk loop they would stay live across it)
    if constexpr (FOLD)
        asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int qc = lane & (T::RPW - 1);   // the lane's row within the wave (MFMA column)
    const int part = lane / T::RPW;       // which part of the row's keys and d the lane holds
    const int h = lane >> 5;
    const int grp = lane >> 4;
    const int s16 = lane & 15;
    const int g = a.group;
    const int r = w * T::RPW + qc;        // tile row
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

    const float c = a.scale_log2;
    // FOLD: this call runs canonical KV chunk fc of a fold item (fold_keys
    // keys per chunk) from a fresh state, by the rules of a split item.
    const int chunk_begin = FOLD ? it.key_begin + fc * it.fold_keys : it.key_begin;
    const int chunk_end = FOLD ? min(it.key_end, chunk_begin + it.fold_keys) : it.key_end;
    const int kb_begin = chunk_begin / T::BK;
    const int kb_end = chunk_end > chunk_begin ? (chunk_end + T::BK - 1) / T::BK : kb_begin;

    const size_t head_off = ((size_t)(PAGED ? 0 : it.kv_row0) * a.num_kv_heads + it.kv_head) * HD;
    const __bf16 *kbase = static_cast<const __bf16 *>(a.k) + head_off;
    const __bf16 *vbase = static_cast<const __bf16 *>(a.v) + head_off;

    // Staging: direct-to-LDS loads.  Wave w, load i fills LDS chunks
    // (NLOAD w + i) * 64 + lane of the tile: key row r = chunk / CPR, position
    // p = chunk % CPR, which holds global chunk p ^ swz(r).  Rows past the end
    // of the request are clamped to its last key: those keys are masked
    // (P = 0 exactly), so the data there is inert.
    const int wu = __builtin_amdgcn_readfirstlane(w);
    // Lane offsets of load i.  The paged head_dim 256 kernel recomputes them
    // at every issue from a fresh lane id (the empty asm keeps the compiler
    // from hoisting them out of the loop): kept live there, they are spilled,
    // and the scratch reload after the K/V loads waits for those loads too
    // (measured: 20 % slower).  The other kernels keep them live, which
    // measured faster for them.
    auto lane_offsets = [&](int ln, int i, int &grow, int &kc, int &vc) __attribute__((always_inline)) {
        const int chunk = (T::NLOAD * wu + i) * 64 + ln;
        const int rr = chunk / T::CPR;
        const int pp = chunk - rr * T::CPR;
        grow = rr;
        kc = 8 * (pp ^ swz_k(rr));
        vc = 8 * (pp ^ swz_v<HD>(rr));
    };
    constexpr bool KEEP_OFFSETS = HD == 128 || !PAGED;
    int grow_[T::NLOAD], kcol[T::NLOAD], vcol[T::NLOAD];
    if constexpr (KEEP_OFFSETS) {
#pragma unroll
        for (int i = 0; i < T::NLOAD; ++i)
            lane_offsets(lane, i, grow_[i], kcol[i], vcol[i]);
    }
    const int kv_stride_i = a.num_kv_heads * HD;
    unsigned koff0[T::NLOAD], voff0[T::NLOAD];
#pragma unroll
    for (int i = 0; i < (HD == 128 ? T::NLOAD : 0); ++i) {
        int gr, kc, vc;
        lane_offsets(lane, i, gr, kc, vc);
        koff0[i] = (unsigned)(gr * kv_stride_i + kc) * 2u;
        voff0[i] = (unsigned)(gr * kv_stride_i + vc) * 2u;
    }
    const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)smem;
    // Paged K/V: a wave's loads of one block move WAVE_ROWS aligned
    // consecutive keys (clamped to the request's last key), so with pages of
    // at least 16 keys they lie in one page: one page id per wave and block,
    // clamped to >= 0 where it is used (padding ids stay harmless).  The id
    // of block kb + 1 is read with an ordinary vector load issued right after
    // block kb's K/V loads: loads complete in order, so the vmcnt wait that
    // ends the iteration covers it and its use at the next issue waits for
    // nothing.  (A scalar load would share lgkmcnt with the LDS reads and
    // turn their graduated waits into full ones.)
    constexpr int WAVE_ROWS = T::NLOAD * 1024 / T::RB;
    static_assert(16 % WAVE_ROWS == 0, "a wave's rows must lie in one 16-key page");
    const int32_t *table_row = PAGED ? a.block_table + (size_t)it.request * a.max_blocks : nullptr;
    const int page_mask = (1 << a.page_shift) - 1;
    int pg_next = 0;
    auto page_id = [&](int kb) __attribute__((always_inline)) {
        const int key0 = min(kb * T::BK + wu * WAVE_ROWS, it.kv_len - 1);
        pg_next = table_row[key0 >> a.page_shift];
    };
    auto issue_loads = [&](int kb, int buf) __attribute__((always_inline)) {
        // page base (paged) or block base in the scalar pointer
        const size_t blk = PAGED ? ((size_t)__builtin_amdgcn_readfirstlane(max(pg_next, 0)) << a.page_shift) * kv_stride_i
                                 : (size_t)kb * T::BK * kv_stride_i;
        const __bf16 *kb_ptr = kbase + blk;
        const __bf16 *vb_ptr = vbase + blk;
        const int last = it.kv_len - 1 - kb * T::BK;
        if (!PAGED && HD == 128 && last >= T::BK - 1) {
            // whole block inside the request: no clamping, constant lane offsets
#pragma unroll
            for (int i = 0; i < T::NLOAD; ++i) {
                const unsigned dk = lds_base + (unsigned)(buf * T::STAGE_BYTES + (T::NLOAD * wu + i) * 1024);
                asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                             :: "s"(dk), "v"(koff0[i]), "s"(kb_ptr) : "memory", "m0");
                asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                             :: "s"(dk + (unsigned)T::TILE_BYTES), "v"(voff0[i]), "s"(vb_ptr)
                             : "memory", "m0");
            }
            return;
        }
        int ln = lane;
        if constexpr (!KEEP_OFFSETS) {
            ln = __lane_id();
            asm volatile("" : "+v"(ln));
#pragma unroll
            for (int i = 0; i < T::NLOAD; ++i)
                lane_offsets(ln, i, grow_[i], kcol[i], vcol[i]);
        }
#pragma unroll
        for (int i = 0; i < T::NLOAD; ++i) {
            int row = min(grow_[i], last);
            if (PAGED)
                row = (kb * T::BK + row) & page_mask;   // in-page row of this lane's key
            const unsigned koff = (unsigned)(row * kv_stride_i + kcol[i]) * 2u;
            const unsigned voff = (unsigned)(row * kv_stride_i + vcol[i]) * 2u;
            const unsigned dk = lds_base + (unsigned)(buf * T::STAGE_BYTES + (T::NLOAD * wu + i) * 1024);
            // global_load_lds_dwordx4: lane l's 16 bytes land at M0 + 16 l.
            // Issued as inline asm so that the compiler does not order the
            // LDS reads of the current buffer behind these loads; the wait
            // for them is the explicit vmcnt wait before the block barrier.
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                         :: "s"(dk), "v"(koff), "s"(kb_ptr) : "memory", "m0");
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                         :: "s"(dk + (unsigned)T::TILE_BYTES), "v"(voff), "s"(vb_ptr)
                         : "memory", "m0");
        }
    };

    // Wait until at most `later` blocks' loads (issued after the one needed
    // next) are still in flight: vmcnt counts this wave's outstanding loads,
    // 2 NLOAD per block.
    auto wait_loads = [&](int later) __attribute__((always_inline)) {
        static_assert(T::STAGES <= 4, "extend the wait cases");
        if (T::STAGES > 3 && later >= 2)
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(4 * T::NLOAD) : "memory");
        else if (T::STAGES > 2 && later >= 1)
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * T::NLOAD) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    // FP8 K/V (e4m3 bytes): each wave moves 8 key rows of K and of V (whole
    // rows of HD bytes, 64 lanes x 16 bytes per load) into its own staging
    // slot after the bf16 stages, then converts the bytes it loaded itself to
    // bf16 (exactly: every e4m3 value is a bf16 value) and writes them into
    // the block's stage in the bf16 layout, so the block computation is
    // unchanged.  The dequantisation scales are folded into the softmax
    // scale (k_scale) and the final normalisation (v_scale).  A wave's 8
    // rows are aligned consecutive keys, so paging keeps one page id per
    // wave and block.  Staging: K of wave w at 8 HD w, V at BK HD + 8 HD w.
    constexpr int F8_W = T::BK / T::NW;        // key rows per wave and block
    constexpr int F8_CPR = HD / 16;            // 16-byte chunks per fp8 row
    constexpr int F8_RPL = 64 / F8_CPR;        // rows per load instruction
    constexpr int F8_NL = F8_W / F8_RPL;       // load instructions per wave and tensor
    static_assert(F8_NL * F8_RPL == F8_W, "fp8 rows must split evenly over a wave's loads");
    auto issue_fp8 = [&](int kb) __attribute__((always_inline)) {
        const int kv_stride_b = a.num_kv_heads * HD;   // bytes between fp8 key rows
        const size_t head_b = ((size_t)(PAGED ? 0 : it.kv_row0) * a.num_kv_heads + it.kv_head) * HD;
        const size_t blk = PAGED ? ((size_t)__builtin_amdgcn_readfirstlane(max(pg_next, 0)) << a.page_shift) * kv_stride_b
                                 : (size_t)kb * T::BK * kv_stride_b;
        const char *kp = static_cast<const char *>(a.k) + head_b + blk;
        const char *vp = static_cast<const char *>(a.v) + head_b + blk;
#pragma unroll
        for (int i = 0; i < F8_NL; ++i) {
            const int f8_row = wu * F8_W + i * F8_RPL + lane / F8_CPR;   // this lane's key row in the block
            const int f8_chunk = lane % F8_CPR;                         // its 16-byte chunk (16 elements)
            int row = min(f8_row, it.kv_len - 1 - kb * T::BK);
            if (PAGED)
                row = (kb * T::BK + row) & page_mask;
            const unsigned off = (unsigned)(row * kv_stride_b + 16 * f8_chunk);
            const unsigned dst = lds_base + (unsigned)(T::STAGES * T::STAGE_BYTES + wu * F8_W * HD + i * 1024);
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                         :: "s"(dst), "v"(off), "s"(kp) : "memory", "m0");
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                         :: "s"(dst + (unsigned)(T::BK * HD)), "v"(off), "s"(vp) : "memory", "m0");
        }
    };
    auto convert_fp8 = [&](int buf) __attribute__((always_inline)) {
        typedef __bf16 bf16x2e __attribute__((ext_vector_type(2)));
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        auto cvt8 = [](unsigned x, unsigned y) __attribute__((always_inline)) {
            u32x4 u;
            u[0] = __builtin_bit_cast(unsigned, (bf16x2e)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
            u[1] = __builtin_bit_cast(unsigned, (bf16x2e)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
            u[2] = __builtin_bit_cast(unsigned, (bf16x2e)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.0f, false));
            u[3] = __builtin_bit_cast(unsigned, (bf16x2e)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.0f, true));
            return __builtin_bit_cast(bf16x8, u);
        };
#pragma unroll
        for (int i = 0; i < F8_NL; ++i) {
            const int f8_row = wu * F8_W + i * F8_RPL + lane / F8_CPR;
            const int f8_chunk = lane % F8_CPR;
            const char *src = smem + T::STAGES * T::STAGE_BYTES + wu * F8_W * HD + i * 1024 + 16 * lane;
            const u32x4 kq = *reinterpret_cast<const u32x4 *>(src);
            const u32x4 vq = *reinterpret_cast<const u32x4 *>(src + T::BK * HD);
            char *Kd = smem + buf * T::STAGE_BYTES + f8_row * T::RB;
            char *Vd = Kd + T::TILE_BYTES;
            const int c0 = 2 * f8_chunk;
            *reinterpret_cast<bf16x8 *>(Kd + 16 * (c0 ^ swz_k(f8_row))) = cvt8(kq[0], kq[1]);
            *reinterpret_cast<bf16x8 *>(Kd + 16 * ((c0 + 1) ^ swz_k(f8_row))) = cvt8(kq[2], kq[3]);
            *reinterpret_cast<bf16x8 *>(Vd + 16 * (c0 ^ swz_v<HD>(f8_row))) = cvt8(vq[0], vq[1]);
            *reinterpret_cast<bf16x8 *>(Vd + 16 * ((c0 + 1) ^ swz_v<HD>(f8_row))) = cvt8(vq[2], vq[3]);
        }
    };

    // The first blocks' K/V loads go out before the Q loads so that the
    // latencies overlap.  Block kb lives in stage kb % STAGES (absolute block
    // parity, so that the unrolled loop below knows every stage at compile
    // time and LDS addresses become per-lane constants plus an immediate).
    const int kb_pre = min(kb_begin + T::STAGES - 1, kb_end);
    auto first_loads = [&]() __attribute__((always_inline)) {
        for (int kb = kb_begin; kb < kb_pre; ++kb) {
            if (PAGED)
                page_id(kb);
            if (FP8)
                issue_fp8(kb);
            else
                issue_loads(kb, kb % T::STAGES);
        }
        if (PAGED && kb_pre < kb_end)
            page_id(kb_pre);
    };
    first_loads();

    WaveState<HD> st;
    constexpr int NQF = R16 ? T::KS16 : T::DS;   // Q fragments
    {
        // lane part `part` holds d (16 or 32) ds + 8 part .. + 7 of its row
        const bf16x8 *qp = reinterpret_cast<const bf16x8 *>(
            static_cast<const __bf16 *>(a.q) + q_row * HD + 8 * part);
#pragma unroll
        for (int ds = 0; ds < NQF; ++ds) {
            if (row_valid) {
                st.qf[ds] = qp[(R16 ? 4 : 2) * ds];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    st.qf[ds][e] = (__bf16)0.0f;
            }
        }
    }
    // Consume the Q fragments here so that the compiler's wait for these
    // loads is placed before the key loop; inside the loop any vmcnt wait
    // would also wait for the K/V prefetch in flight.
#pragma unroll
    for (int ds = 0; ds < NQF; ++ds)
        asm volatile("" :: "v"(st.qf[ds]));
    constexpr int NACC = R16 ? 4 * T::DT16 : 16 * T::DB;   // accumulator floats per lane
    static_assert(NACC * sizeof(float) == sizeof(st.acc), "accumulator layout");
    auto acc_at = [&](int i) __attribute__((always_inline)) -> float {
        if constexpr (R16)
            return st.acc[i / 4][i % 4];
        else
            return st.acc[i / 16][i % 16];
    };
    auto start = [&]() __attribute__((always_inline)) {
        if constexpr (R16) {
#pragma unroll
            for (int dt = 0; dt < T::DT16; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st.acc[dt][i] = 0.0f;
        } else {
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    st.acc[db][i] = 0.0f;
        }
        st.m = -INFINITY;
        st.l = 0.0f;
        wait_loads(kb_pre - kb_begin - 1);
        if (FP8 && kb_begin < kb_end)
            convert_fp8(kb_begin % T::STAGES);
        __syncthreads();
    };
    start();

    // Blocks below the first row's causal limit need no mask; they come
    // first.  The rest (diagonal and KV tail) are masked.  Each range runs as
    // its own loop over one block_step variant.
    const int kb_mask = min(max(it.lim_first / T::BK, kb_begin), kb_end);
    // head_dim 128: a wave whose 32 rows all lie past the tile's rows (decode
    // tiles, the last tile of a request) only takes part in the loads and
    // barriers; it skips the block computation and leaves its SIMD to the
    // other workgroup on the CU (FP8 decode 14 % faster).  Uniform per wave.
    // (At head_dim 256, one workgroup per CU, the branch only costs spills.)
    const bool wave_rows = w * T::RPW < it.n_tok * g;
    // Tiles whose first row sees at most kHiLoKeys keys (rows with few keys,
    // where single keys carry much of the softmax) split P on every block.
    // Other final items round P to bf16 and are recomputed with P split on
    // every block when the result holds an element with |O| >=
    // kRecomputeAbsO (below); partial states of split-KV tiles cannot be
    // recomputed later, so they split P per block by the running-sum test.
    // Fold items follow the rules of split items (slot >= 0).  Their slot is
    // made opaque so that the key loop is compiled as for any item (known
    // at compile time, the specialised loop needs more registers at head_dim 256).
    int slot_rt = it.slot;
    if constexpr (FOLD)
        asm volatile("" : "+s"(slot_rt));
    const bool final_item = slot_rt < 0;
    const bool force = it.lim_first <= kHiLoKeys;
    const bool trig = !final_item;
    const float kappa = trig ? kHiLoFracPartial / (1.0f - kHiLoFracPartial) : INFINITY;
    auto run = [&](auto mask_tag, auto force_tag, int kb_from, int kb_to) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr bool FORCE = decltype(force_tag)::value;
        static_assert(T::STAGES == 2, "the loops assume two stages");
        auto step = [&](int kb, auto buf_tag) __attribute__((always_inline)) {
            constexpr int BUF = decltype(buf_tag)::value;
            if (kb + 1 < kb_end) {
                if (FP8)
                    issue_fp8(kb + 1);
                else
                    issue_loads(kb + 1, BUF ^ 1);
                // the page ids of the block loaded next iteration
                if (PAGED && kb + 2 < kb_end)
                    page_id(kb + 2);
            }
            const char *Ks = smem + BUF * T::STAGE_BYTES;
            const char *Vs = Ks + T::TILE_BYTES;
            const int thr = lim_row - kb * T::BK - 4 * part;
            if constexpr (R16)
                block_step16<HD, POS_SCALE, MASK, FORCE>(st, Ks, Vs, c, thr, row_valid, trig, kappa, qc, part);
            else if (HD != 128 || wave_rows)
                block_step<HD, POS_SCALE, MASK, FORCE>(st, Ks, Vs, c, thr, row_valid, trig, kappa,
                                                       qc, h, grp, s16);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // block kb + 1 has landed
            if (FP8 && kb + 1 < kb_end)
                convert_fp8(BUF ^ 1);
            __syncthreads();
        };
        int kb = kb_from;
        if (kb < kb_to && (kb & 1)) {
            step(kb, std::integral_constant<int, 1>{});
            ++kb;
        }
        for (; kb + 1 < kb_to; kb += 2) {
            step(kb, std::integral_constant<int, 0>{});
            step(kb + 1, std::integral_constant<int, 1>{});
        }
        if (kb < kb_to)
            step(kb, std::integral_constant<int, 0>{});
    };
    auto run_forced = [&]() __attribute__((always_inline)) {
        run(std::false_type{}, std::true_type{}, kb_begin, kb_mask);
        run(std::true_type{}, std::true_type{}, kb_mask, kb_end);
    };
    auto set_acc = [&](int i, float x) __attribute__((always_inline)) {
        if constexpr (R16)
            st.acc[i / 4][i % 4] = x;
        else
            st.acc[i / 16][i % 16] = x;
    };
    // Fold items, at the end of chunk fc: the chunk's normalised state (as a
    // split item writes it) becomes the running state (first chunk) or is
    // folded into it.  The running state lives in the item's slot: outputs
    // in part_o, each lane reading back only what it wrote itself, and the
    // log-sum-exp in part_lse, written by every lane of the row (the same
    // value).  After the last chunk the folded outputs replace the
    // accumulators and the folded log-sum-exp is returned.  Lane layout:
    // 4 consecutive floats of row r per group of 4 accumulators.
    constexpr int FOLD_LOADS = 4;
    auto fold_chunk = [&](bool first, auto last_tag) __attribute__((always_inline)) {
        constexpr bool LAST = decltype(last_tag)::value;
        const float lt = row_sum<HD>(st.l);
        const float inv = lt > 0.0f ? (FP8 ? a.v_scale : 1.0f) / lt : 0.0f;
        const float lse_c = lt > 0.0f ? st.m + log2f(lt) : -INFINITY;
        float *orow = a.part_o + ((size_t)it.slot * kTileRows + r) * HD;
        float *lrow = a.part_lse + (size_t)it.slot * kTileRows + r;
        const float lse_run = first ? -INFINITY : *lrow;
        const FoldWeights fw = fold_weights(lse_run, lse_c);
#pragma unroll
        for (int gq = 0; gq < NACC / 4; ++gq) {
            const int d0 = R16 ? 16 * gq + 4 * part : 32 * (gq / 4) + 8 * (gq % 4) + 4 * h;
            float4 *p4 = reinterpret_cast<float4 *>(orow + d0);
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = acc_at(4 * gq + e) * inv;
            if (!first) {
                const float4 x = *p4;
                o[0] = fold_value(fw, x.x, o[0]);
                o[1] = fold_value(fw, x.y, o[1]);
                o[2] = fold_value(fw, x.z, o[2]);
                o[3] = fold_value(fw, x.w, o[3]);
            }
            if constexpr (LAST) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    set_acc(4 * gq + e, o[e]);
            } else {
                *p4 = make_float4(o[0], o[1], o[2], o[3]);
            }
            // at most FOLD_LOADS float4 loads in flight
            if (gq % FOLD_LOADS == FOLD_LOADS - 1)
                asm volatile("" ::: "memory");
        }
        const float lse_new = first ? lse_c : fw.lse;
        if (!LAST)
            *lrow = lse_new;
        return lse_new;
    };
    if (force) {
        run_forced();
    } else {
        run(std::false_type{}, std::false_type{}, kb_begin, kb_mask);
        run(std::true_type{}, std::false_type{}, kb_mask, kb_end);
        if (final_item) {
            // Recompute?  A wave votes for it when one of its valid rows has
            // an output element with |O| >= kRecomputeAbsO; the flags of the
            // waves are combined through LDS (after the staging area,
            // which the epilogue reuses), and the workgroup recomputes
            // together (the K/V staging is shared).
            bool redo = false;
            {
                const float lt = row_sum<HD>(st.l);
                float omax = 0.0f;
#pragma unroll
                for (int i = 0; i < NACC; ++i)
                    omax = fmaxf(omax, fabsf(acc_at(i)));
                if (FP8)
                    omax *= fabsf(a.v_scale);
                redo = row_valid && lt > 0.0f && omax >= kRecomputeAbsO * lt;
            }
            int *flags = reinterpret_cast<int *>(smem + Tile<HD>::LDS_BYTES + (FP8 ? 2 * T::BK * HD : 0));
            const bool wave_redo = __any(redo);
            if (lane == 0)
                flags[w] = wave_redo ? 1 : 0;
            __syncthreads();
            int any_redo = 0;
#pragma unroll
            for (int i = 0; i < T::NW / 4; ++i) {
                const int4 f = reinterpret_cast<const int4 *>(flags)[i];
                any_redo |= f.x | f.y | f.z | f.w;
            }
            if (any_redo) {
                first_loads();
                start();
                run_forced();
            }
        }
    }
    float lse_fold = 0.0f;
    if constexpr (FOLD) {
        // the last block's barrier has freed the stages for the next chunk
        if (chunk_end < it.key_end) {
            fold_chunk(fc == 0, std::false_type{});
            return;
        }
        lse_fold = fold_chunk(fc == 0, std::true_type{});
    }

    // ---- epilogue ----
    const float lt = row_sum<HD>(st.l);
    // fold items hold the folded (already normalised) outputs
    const float inv = FOLD ? 1.0f : lt > 0.0f ? (FP8 ? a.v_scale : 1.0f) / lt : 0.0f;
    const float lse2 = FOLD ? lse_fold : lt > 0.0f ? st.m + log2f(lt) : -INFINITY;
    const bool write_final = FOLD || it.slot < 0;
    // The outputs go out through LDS (the K/V stages are free after the last
    // block barrier; each wave uses its own region): the wave writes its
    // O^T fragments as rows, 16-byte chunk c of row r at position
    // c ^ (r mod chunks-per-row), reads back whole 16-byte row chunks, and
    // stores full row segments, so that consecutive lanes write consecutive
    // bytes (the g heads of a token are adjacent rows of O).
    const float inv_g = 1.0f / (float)g;
    auto row_out = [&](int rr, size_t &orow) __attribute__((always_inline)) {
        const int R = w * T::RPW + rr;
        const int tk = (int)(((float)R + 0.5f) * inv_g);
        orow = (size_t)(it.q_tok0 + tk) * a.num_qo_heads + it.kv_head * g + (R - tk * g);
        return tk < it.n_tok;
    };
    if (R16 && write_final) {
        // 16-row waves: acc[dt][i] is d = 16 dt + 4 part + i of row qc, so a
        // 16-byte chunk 2 dt + part / 2 is written by lanes part and part ^ 1
        constexpr int CPR = T::CPR;
        constexpr int RPI = 64 / CPR;
        char *wl = smem + w * (T::RPW * T::RB);
#pragma unroll
        for (int dt = 0; dt < T::DT16; ++dt) {
            bf16x4 ov;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ov[e] = (__bf16)(acc_at(4 * dt + e) * inv);
            const int cc = 2 * dt + (part >> 1);
            *reinterpret_cast<bf16x4 *>(wl + qc * T::RB + 16 * (cc ^ (qc & (CPR - 1))) + 8 * (part & 1)) = ov;
        }
#pragma unroll
        for (int i = 0; i < T::RPW / RPI; ++i) {
            const int rr = RPI * i + lane / CPR;
            const int cc = lane % CPR;
            const bf16x8 x = *reinterpret_cast<const bf16x8 *>(wl + rr * T::RB + 16 * (cc ^ (rr & (CPR - 1))));
            size_t orow;
            if (row_out(rr, orow))
                *reinterpret_cast<bf16x8 *>(static_cast<__bf16 *>(a.o) + orow * HD + 8 * cc) = x;
        }
        if (row_valid && part == 0 && a.lse != nullptr)
            a.lse[q_row] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
    } else if (R16) {
        // fp32 partial state in two passes over d: d tiles 8 pass .. + 7,
        // chunk 4 (dt - 8 pass) + part of a 512-byte row
        constexpr int DTP = T::DT16 / 2;
        constexpr int CPRF = DTP * 4;
        constexpr int RPIF = 64 / CPRF;
        char *wl = smem + w * (T::RPW * CPRF * 16);
        float *pbase = a.part_o + (size_t)it.slot * kTileRows * HD;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int dtl = 0; dtl < DTP; ++dtl) {
                const int dt = pass * DTP + dtl;
                float4 ov;
                ov.x = acc_at(4 * dt + 0) * inv;
                ov.y = acc_at(4 * dt + 1) * inv;
                ov.z = acc_at(4 * dt + 2) * inv;
                ov.w = acc_at(4 * dt + 3) * inv;
                const int cc = 4 * dtl + part;
                *reinterpret_cast<float4 *>(wl + qc * (CPRF * 16) + 16 * (cc ^ (qc & (CPRF - 1)))) = ov;
            }
#pragma unroll
            for (int i = 0; i < T::RPW / RPIF; ++i) {
                const int rr = RPIF * i + lane / CPRF;
                const int cc = lane % CPRF;
                const float4 x = *reinterpret_cast<const float4 *>(
                    wl + rr * (CPRF * 16) + 16 * (cc ^ (rr & (CPRF - 1))));
                size_t orow;
                if (row_out(rr, orow))
                    *reinterpret_cast<float4 *>(pbase + (size_t)(w * T::RPW + rr) * HD + pass * DTP * 16 + 4 * cc) = x;
            }
        }
        if (row_valid && part == 0)
            a.part_lse[(size_t)it.slot * kTileRows + r] = lse2;
    } else if (write_final) {
        constexpr int CPR = T::CPR;          // 16-byte chunks per bf16 row
        constexpr int RPI = 64 / CPR;        // rows per read instruction
        char *wl = smem + w * (32 * T::RB);
        // Lane half h holds bytes 8 h .. 8 h + 7 of every 16-byte chunk of its
        // row; one permlane32 swap per dword pairs the halves, so that the
        // lower lane writes chunk 4 db + 2 p and the upper lane chunk
        // 4 db + 2 p + 1 whole (16-byte writes, no bank conflicts).
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                bf16x4 ox, oy;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ox[e] = (__bf16)(st.acc[db][8 * pp + e] * inv);
                    oy[e] = (__bf16)(st.acc[db][8 * pp + 4 + e] * inv);
                }
                const u32x2 x2 = __builtin_bit_cast(u32x2, ox);
                const u32x2 y2 = __builtin_bit_cast(u32x2, oy);
                auto r0 = __builtin_amdgcn_permlane32_swap(x2[0], y2[0], false, false);
                auto r1 = __builtin_amdgcn_permlane32_swap(x2[1], y2[1], false, false);
                u32x4 ch;
                ch[0] = r0[0];
                ch[1] = r1[0];
                ch[2] = r0[1];
                ch[3] = r1[1];
                const int cc = 4 * db + 2 * pp + h;
                *reinterpret_cast<u32x4 *>(wl + qc * T::RB + 16 * (cc ^ (qc & (CPR - 1)))) = ch;
            }
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int rr = RPI * i + lane / CPR;
            const int cc = lane % CPR;
            const bf16x8 x = *reinterpret_cast<const bf16x8 *>(wl + rr * T::RB + 16 * (cc ^ (rr & (CPR - 1))));
            size_t orow;
            if (row_out(rr, orow))
                *reinterpret_cast<bf16x8 *>(static_cast<__bf16 *>(a.o) + orow * HD + 8 * cc) = x;
        }
        if (row_valid && h == 0 && a.lse != nullptr)
            a.lse[q_row] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
    } else {
        // fp32 partial state of the tile's rows, in two passes over d
        constexpr int DBP = T::DB / 2;       // d blocks per pass
        constexpr int CPRF = DBP * 8;        // 16-byte chunks per row and pass
        constexpr int RPIF = 64 / CPRF;
        char *wl = smem + w * (32 * CPRF * 16);
        float *pbase = a.part_o + (size_t)it.slot * kTileRows * HD;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int dbl = 0; dbl < DBP; ++dbl)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int db = pass * DBP + dbl;
                    float4 ov;
                    ov.x = st.acc[db][4 * jj + 0] * inv;
                    ov.y = st.acc[db][4 * jj + 1] * inv;
                    ov.z = st.acc[db][4 * jj + 2] * inv;
                    ov.w = st.acc[db][4 * jj + 3] * inv;
                    const int cc = 8 * dbl + 2 * jj + h;
                    *reinterpret_cast<float4 *>(wl + qc * (CPRF * 16) + 16 * (cc ^ (qc & (CPRF - 1)))) = ov;
                }
#pragma unroll
            for (int i = 0; i < 32 / RPIF; ++i) {
                const int rr = RPIF * i + lane / CPRF;
                const int cc = lane % CPRF;
                const float4 x = *reinterpret_cast<const float4 *>(
                    wl + rr * (CPRF * 16) + 16 * (cc ^ (rr & (CPRF - 1))));
                size_t orow;
                if (row_out(rr, orow))
                    *reinterpret_cast<float4 *>(pbase + (size_t)(w * 32 + rr) * HD + pass * DBP * 32 + 4 * cc) = x;
            }
        }
        if (row_valid && h == 0)
            a.part_lse[(size_t)it.slot * kTileRows + r] = lse2;
    }
}

// FOLDK: the instance that also runs fold items (it is built in its own
// translation unit; the extra path costs registers, so plans without fold
// items launch the plain instance).
template <int HD, bool PAGED, bool FP8, bool FOLDK>
__global__ __launch_bounds__(Tile<HD>::THREADS, HD == 128 ? 2 : 1) void tile_kernel(TileArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const Item it = a.items[blockIdx.x];
    if (it.n_tok == 0)
        return;  // padding item of the launch order
    if constexpr (FOLDK) {
        if (it.fold_keys > 0) {
            // in-workgroup chunk folding: the tile's canonical KV chunks in
            // order (the running state is carried in the item's slot)
            const int n = (it.key_end - it.key_begin + it.fold_keys - 1) / it.fold_keys;
            for (int fc = 0; fc < n; ++fc) {
                if (a.scale_log2 > 0.0f)
                    tile_body<HD, true, PAGED, FP8, true>(a, it, smem, fc);
                else
                    tile_body<HD, false, PAGED, FP8, true>(a, it, smem, fc);
            }
            return;
        }
    }
    if (a.scale_log2 > 0.0f)
        tile_body<HD, true, PAGED, FP8, false>(a, it, smem, 0);
    else
        tile_body<HD, false, PAGED, FP8, false>(a, it, smem, 0);
}

// dynamic LDS of a tile kernel instance: the K/V stages, the fp8 staging
// slots, and the per-wave recompute flags
template <int HD, bool FP8>
constexpr int tile_lds_bytes() { return Tile<HD>::LDS_BYTES + (FP8 ? 2 * Tile<HD>::BK * HD : 0) + 4 * Tile<HD>::NW; }

#if !RP_TILE_FOLD
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
            const FoldWeights fw = fold_weights(lse_run, lse_c);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o_run[e] = fold_value(fw, o_run[e], o_c[e]);
            lse_run = fw.lse;
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

#endif

template <int HD, bool PAGED, bool FP8>
int launch_tile(const TileArgs &args, int64_t num_items, hipStream_t stream)
{
    constexpr bool FOLDK = RP_TILE_FOLD != 0;
    constexpr int lds = tile_lds_bytes<HD, FP8>();
    const void *fn = reinterpret_cast<const void *>(&tile_kernel<HD, PAGED, FP8, FOLDK>);
    // The dynamic-LDS limit is a per-device function attribute: set it once
    // per device (devices beyond 64 set it at every launch).
    static std::atomic<unsigned long long> attr_devices{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return (int)e;
    const unsigned long long bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
    if (bit == 0 || (attr_devices.load(std::memory_order_acquire) & bit) == 0) {
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess)
            return (int)e;
        attr_devices.fetch_or(bit, std::memory_order_release);
    }
    auto kernel = tile_kernel<HD, PAGED, FP8, FOLDK>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)num_items), dim3(Tile<HD>::THREADS), lds, stream, args);
    return (int)hipGetLastError();
}

}  // namespace

#if RP_TILE_FOLD
int launch_tile_fold_kernel(int head_dim, bool paged, bool fp8, const TileArgs &args, int64_t num_items,
                            void *stream)
#else
int launch_tile_kernel(int head_dim, bool paged, bool fp8, bool fold, const TileArgs &args,
                       int64_t num_items, void *stream)
#endif
{
#if !RP_TILE_FOLD
    if (fold)
        return launch_tile_fold_kernel(head_dim, paged, fp8, args, num_items, stream);
#endif
    if (num_items <= 0)
        return (int)hipSuccess;
    if (num_items > INT_MAX)
        return (int)hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (head_dim == 128 && fp8)
        return paged ? launch_tile<128, true, true>(args, num_items, s)
                     : launch_tile<128, false, true>(args, num_items, s);
    if (head_dim == 128)
        return paged ? launch_tile<128, true, false>(args, num_items, s)
                     : launch_tile<128, false, false>(args, num_items, s);
    if (head_dim == 256 && fp8)
        return paged ? launch_tile<256, true, true>(args, num_items, s)
                     : launch_tile<256, false, true>(args, num_items, s);
    if (head_dim == 256)
        return paged ? launch_tile<256, true, false>(args, num_items, s)
                     : launch_tile<256, false, false>(args, num_items, s);
    return (int)hipErrorInvalidValue;
}

#if !RP_TILE_FOLD
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

#endif

}  // namespace rp
