// Tree-masked softmax attention over a packed pass, for gfx950 (MI355X).
//
// Source: "Serving 0.88M TPS from Two RTXs and Mac Minis", section "The
// Workload": Span-1 is a hybrid of linear-attention layers and a few
// softmax-attention layers, and a branch attends to its own view but never
// to another branch; section "Long Requests": the view cache also holds the
// K/V of the softmax layers, so a branch shard attends to cached view keys and
// values.  Per head and token t, over the attend set A(t) (t's own segment up
// to and including t, plus the whole parent view for a branch):
//     o_t = sum_{u in A(t)} exp(s_tu - m_t) v_u / sum_{u in A(t)} exp(s_tu - m_t),
//     s_tu = scale * q_t . k_u,   m_t = max_u s_tu.
//
// One workgroup of 4 waves per (query block of <= 64 tokens, head).  It walks
// the block's keys in 64-key blocks -- first the parent view's (from the pass
// or from the external K/V arrays), then its own segment's up to and
// including the query block -- keeping for every query a running maximum, a
// running sum and the unnormalised output (the usual online softmax).  The
// four waves split each 64 x 64 (queries x keys) block into 2 x 2 tiles:
// wave w owns queries 32 (w % 2) .. + 31 against keys 32 (w / 2) .. + 31 of
// every key block, with a running maximum and sum of its own; the two key
// halves of a query are merged after the last block (the softmax of a union
// of key sets from the parts' maxima and sums).  MFMA orientation, as in the
// scan's output kernel: scores are computed transposed, S^T = K Q^T (A = K
// rows from LDS, B = Q^T fragments held in registers), so each lane owns one
// query of a tile (its column) and 8 keys of its half; exponentiated scores,
// packed to bf16, are the B operand of O^T += V^T P^T directly from the
// accumulator layout.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <type_traits>

#include "linattn.h"
#include "tiles.h"

namespace {

struct AttnItem {
    int q0, nq, seg0, view0, view_len, view_src, pad0, pad1;
};

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes that hold
// one query's scores), with the gfx950 lane-swap instructions: each swap
// leaves a lane's own value in one result and its partner's in the other.
__device__ __forceinline__ float max_over_groups(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t uy = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane16_swap(uy, uy, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// QT query tiles of 16 per wave; KH key parts per 64-key block.  With
// KH = 1 a wave takes 16 QT queries against every key (4 / QT waves per
// 64-query item); with KH = 2 the four waves form 2 x 2 tiles of 32 queries
// x 32 keys: a wave reads half of each K and V block from LDS for twice the
// queries, keeps its own running maximum and sums over its keys, and the two
// key halves of a query are merged once, after the last block.  Every K and
// V fragment a wave reads from LDS feeds QT MFMAs.
template <int D, int QT, int KH>
__global__ __launch_bounds__(64 * KH * (4 / QT))
__attribute__((amdgpu_waves_per_eu(KH == 2 && D == 64 ? 4 : 1))) void attn_kernel_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ ext_k,
    const uint16_t* __restrict__ ext_v, const AttnItem* __restrict__ items,
    uint16_t* __restrict__ out, int H, float scale_log2) {
    static_assert(KH == 1 || (KH == 2 && QT == 2), "key halves pair with 32-query waves");
    constexpr int NQG = 4 / QT;          // query groups (waves per key part)
    constexpr int NT = 64 * KH * NQG;
    constexpr int NUB = 4 / KH;          // 16-key tiles of a block per wave
    constexpr int R = 4, NKS = D / 32, NVB = D / 16;
    using ST = Stage<D, R>;
    constexpr int NPER = KVStage<D, D, R, NT>::NPER;
    constexpr int LDR = ST::LDR;
    constexpr int LDV = ST::template LDV<D>;
    // K block then V block, both row-major; after the last block the key
    // halves' partial results are merged through the same memory
    constexpr int kMergeFloats = NQG * (QT * NVB * 64 * 4 + 2 * QT * 64);
    static_assert(KH == 1 || kMergeFloats * 4 <= kChunk * (LDR + LDV) * 2, "merge fits");
    __shared__ __attribute__((aligned(16))) uint16_t sKV[kChunk * (LDR + LDV)];
    uint16_t* sK = sKV;
    uint16_t* sV = sKV + kChunk * LDR;

    const int h = blockIdx.x % H;
    const AttnItem it = items[blockIdx.x / H];
    const int w = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
    const int qg = w % NQG, kh = w / NQG;   // query group, key part (wave-uniform)
    // this lane's queries within the block: tile t holds trow0 + 16 t
    const int trow0 = qg * 16 * QT + c16;
    const int64_t row_elems = int64_t(H) * D;

    // key blocks: the parent view's, then the segment's own up to the query
    // block (q0 - seg0 is a multiple of 64, so the last own block is the
    // query block itself: the diagonal)
    const int n_view_blk = (it.view_len + kChunk - 1) / kChunk;
    const int n_own_blk = (it.q0 - it.seg0) / kChunk + 1;
    const int nkb = n_view_blk + n_own_blk;
    const bool ext_view = it.view_src == LA_ATTN_EXT_VIEW;

    // Q^T fragments (B operand): lane holds q[trow][ks*32 + 8g .. +7]
    u32x4 qf[QT][NKS];
    {
        const auto rq = chunk_rsrc(q, int64_t(it.q0) * row_elems, 2, it.nq, H, D);
#pragma unroll
        for (int t = 0; t < QT; ++t)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                qf[t][ks] = buf_load16(
                    rq, uint32_t((((trow0 + 16 * t) * H + h) * D + ks * 32 + 8 * g) * 2));
    }

    // source of key block b (wave-uniform): token offset and valid rows
    auto block_src = [&](int b, int64_t& tok, int& rows, bool& from_ext) {
        if (b < n_view_blk) {
            tok = int64_t(it.view0) + int64_t(b) * kChunk;
            rows = min(kChunk, it.view_len - b * kChunk);
            from_ext = ext_view;
        } else {
            const int j = b - n_view_blk;
            tok = int64_t(it.seg0) + int64_t(j) * kChunk;
            rows = j == n_own_blk - 1 ? it.nq : kChunk;
            from_ext = false;
        }
        if (b >= nkb) rows = 0;                       // past the end: empty window
        if (from_ext && ext_k == nullptr) rows = 0;   // no external arrays given
    };
    // This thread's share of a key block's staging, the same for every block:
    // piece i is R tokens x 8 features of K or of V (wave-uniform choice), at
    // byte goff[i] of the block's window (+ one head row per token) and at
    // element loff[i] of its LDS tile (+ one tile row per token).
    using KS = KVStage<D, D, R, NT>;
    BlkR<R> kv[NPER];
    uint32_t goff[NPER];
    int loff[NPER];
    bool isv[NPER];
    {
        const int wbase = w * 64;
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
            const int b0 = wbase + i * NT;   // wave-uniform
            isv[i] = b0 >= KS::NBK;
            const int wb = (isv[i] ? b0 - KS::NBK : b0) + lane;
            const int rg = wb / KS::NCGK, cg = wb % KS::NCGK;
            goff[i] = uint32_t((((rg * R) * H + h) * D + cg * 8) * 2);
            loff[i] = (rg * R) * (isv[i] ? LDV : LDR) + cg * 8;
        }
    }
    const uint32_t row_bytes = uint32_t(H) * D * 2;
    auto load = [&](int b) {
        int64_t tok;
        int rows;
        bool fe;
        block_src(b, tok, rows, fe);
        const auto rk = chunk_rsrc(fe ? ext_k : k, tok * row_elems, 2, rows, H, D);
        const auto rv = chunk_rsrc(fe ? ext_v : v, tok * row_elems, 2, rows, H, D);
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
            if constexpr (NPER * NT > KS::NBK + KS::NBV)
                if (w * 64 + i * NT >= KS::NBK + KS::NBV) break;
#pragma unroll
            for (int r = 0; r < R; ++r)
                kv[i].r[r] = buf_load16(isv[i] ? rv : rk, goff[i] + uint32_t(r) * row_bytes);
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
            if constexpr (NPER * NT > KS::NBK + KS::NBV)
                if (w * 64 + i * NT >= KS::NBK + KS::NBV) break;
            uint16_t* dst = (isv[i] ? sV : sK) + loff[i];
            const int ld = isv[i] ? LDV : LDR;
#pragma unroll
            for (int r = 0; r < R; ++r) *reinterpret_cast<u32x4*>(dst + r * ld) = kv[i].r[r];
        }
    };

    // Online softmax with a lazily moved reference maximum: a lane's weights
    // are exp2((s - m) * scale_log2) against a reference m that is raised
    // only when a block's maximum exceeds it by more than 2^kLazy in weight
    // (then the running sums are rescaled); otherwise weights up to 2^kLazy
    // are accumulated as they are.  The final division by the running sum
    // cancels the reference, so the result is the softmax for any m.  The
    // reference is kept in the exponent's units (score * scale_log2) and
    // starts at kNoRef, a finite value below any scaled score: the first
    // block with a key raises it, a lane with no key so far gets weights
    // exp2(-inf) = 0, and no test for "no reference yet" is needed.
    constexpr float kLazy = 8.f;
    constexpr float kNoRef = -1e30f;
    float m[QT];           // reference of each of this lane's queries (log2 units)
    f32x4 acc[QT][NVB];    // O^T tiles: lane holds O[trow][x*16 + 4g + j]
    // running sums of the weights, as one more O^T tile whose A operand is
    // all ones: every row of it holds the sum for the lane's query (column),
    // in the bf16-rounded weights that also multiply V
    f32x4 accl[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        m[t] = kNoRef;
        accl[t] = zero4();
#pragma unroll
        for (int x = 0; x < NVB; ++x) acc[t][x] = zero4();
    }
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

    // one key block: scores, online softmax update, O^T += V^T P^T.  Only the
    // diagonal block and a ragged last view block need the mask (MASKED).
    auto block = [&](int rows, bool diag, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        // S^T tiles (ub = key tile): lane holds s[u = ub*16 + 4g + j][trow]
        // (this wave's key tiles: kh * NUB + ub)
        f32x4 s[QT][NUB];
#pragma unroll
        for (int t = 0; t < QT; ++t)
#pragma unroll
            for (int ub = 0; ub < NUB; ++ub) s[t][ub] = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4 kf[NUB];
#pragma unroll
            for (int ub = 0; ub < NUB; ++ub)
                kf[ub] = lds_u32x4(sK + ((kh * NUB + ub) * 16 + c16) * LDR + ks * 32 + 8 * g);
#pragma unroll
            for (int t = 0; t < QT; ++t)
#pragma unroll
                for (int ub = 0; ub < NUB; ++ub)
                    s[t][ub] = mfma_bf16(kf[ub], qf[t][ks], s[t][ub]);
        }
        bool any_raise = false;
        float bm[QT];
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            float mx = -INFINITY;
#pragma unroll
            for (int ub = 0; ub < NUB; ++ub)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (MASKED) {
                        const int u = (kh * NUB + ub) * 16 + 4 * g + j;
                        if (!(u < rows && (!diag || u <= trow0 + 16 * t))) s[t][ub][j] = -INFINITY;
                    }
                    mx = fmaxf(mx, s[t][ub][j]);
                }
            bm[t] = max_over_groups(mx);
            // raise the reference where the block's maximum is more than
            // 2^kLazy above it in weight (always from kNoRef; never for a
            // block with no key of this query, whose maximum is -inf)
            any_raise |= fmaf(bm[t], scale_log2, -m[t]) > kLazy;
        }
        if (__builtin_amdgcn_ballot_w64(any_raise) != 0) {   // wave-uniform
#pragma unroll
            for (int t = 0; t < QT; ++t) {
                const bool raise = fmaf(bm[t], scale_log2, -m[t]) > kLazy;
                const float mn = raise ? bm[t] * scale_log2 : m[t];
                // from kNoRef: exp2(-huge) = 0, and the sums are zero anyway
                const float alpha = __builtin_amdgcn_exp2f(m[t] - mn);
#pragma unroll
                for (int x = 0; x < NVB; ++x) acc[t][x] *= alpha;
                accl[t][0] *= alpha;
                m[t] = mn;
            }
        }
        // weights exp2(score * scale_log2 - m): at most 2^kLazy, and 0 for
        // masked scores (-inf) whatever the reference
        u32x2 pb[QT][NUB];
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            const float nb = -m[t];
#pragma unroll
            for (int ub = 0; ub < NUB; ++ub) {
                float p[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)   // exp2(-inf) = 0
                    p[j] = __builtin_amdgcn_exp2f(fmaf(s[t][ub][j], scale_log2, nb));
                pb[t][ub] = u32x2{cvt_bf2(p[0], p[1]), cvt_bf2(p[2], p[3])};
            }
        }
        // O^T += V^T P^T; k-slots (g, i) -> key u = (2pp + i/4)*16 + 4g + i%4
#pragma unroll
        for (int pp = 0; pp < NUB / 2; ++pp) {
            u32x4 av[NVB];
#pragma unroll
            for (int x = 0; x < NVB; ++x)
                av[x] = tr_frag(sV, LDV, x * 16, kh * (NUB / 2) + pp, g, c16);
#pragma unroll
            for (int t = 0; t < QT; ++t) {
                const u32x4 bp = cat2(pb[t][2 * pp], pb[t][2 * pp + 1]);
#pragma unroll
                for (int x = 0; x < NVB; ++x) acc[t][x] = mfma_bf16(av[x], bp, acc[t][x]);
                accl[t] = mfma_bf16(ones, bp, accl[t]);
            }
        }
    };

    // Processing order: the full key blocks first (view blocks, then the
    // segment's own blocks before the diagonal), then the blocks that need
    // the mask: a ragged last view block and the diagonal.  Each group runs
    // one copy of the block body.
    const int n_full_view = it.view_len / kChunk;
    const bool view_ragged = n_full_view < n_view_blk;
    const int n_full = n_full_view + n_own_blk - 1;
    auto order = [&](int i) -> int {   // processing index -> key block (as in block_src)
        if (i < n_full_view) return i;
        if (i < n_full) return n_view_blk + (i - n_full_view);
        if (view_ragged && i == n_full) return n_view_blk - 1;
        return i < nkb ? nkb - 1 : nkb;   // nkb: past the end, an empty window
    };
    load(order(0));
    int i = 0;
    for (; i < n_full; ++i) {
        stage();
        __syncthreads();
        load(order(i + 1));
        block(kChunk, false, std::false_type{});
        __syncthreads();
    }
    for (; i < nkb; ++i) {
        stage();
        __syncthreads();
        load(order(i + 1));
        const int b = order(i);
        int64_t tok;
        int rows;
        bool fe;
        block_src(b, tok, rows, fe);
        block(rows, b == nkb - 1, std::true_type{});
        __syncthreads();
    }
    // the lane's position again, opaque to the compiler, so that the offsets
    // below are recomputed here rather than kept in registers over the loops
    int lane_e = int(threadIdx.x);
    asm volatile("" : "+v"(lane_e));
    lane_e &= 63;
    const int trow_e = qg * 16 * QT + (lane_e & 15), g_e = lane_e >> 4;
    if constexpr (KH == 2) {
        // merge the key halves: the second half's waves leave their reference
        // maxima, sums and unnormalised outputs in LDS (the loop ended with a
        // barrier, so the K / V tiles are free); the first half's waves
        // rescale both to the larger reference and add
        float* mg = reinterpret_cast<float*>(sKV) + qg * (QT * NVB * 64 * 4 + 2 * QT * 64);
        f32x4* macc = reinterpret_cast<f32x4*>(mg);
        float* mm = mg + QT * NVB * 64 * 4;
        float* ml = mm + QT * 64;
        if (kh == 1) {
#pragma unroll
            for (int t = 0; t < QT; ++t) {
#pragma unroll
                for (int x = 0; x < NVB; ++x) macc[(t * NVB + x) * 64 + lane_e] = acc[t][x];
                mm[t * 64 + lane_e] = m[t];
                ml[t * 64 + lane_e] = accl[t][0];
            }
        }
        __syncthreads();
        if (kh == 1) return;
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            // the first half holds a key of every query (the diagonal
            // block's first key), so its reference is a real score; a second
            // half with no key kept kNoRef and weighs exp2(-huge) = 0
            const float m1 = mm[t * 64 + lane_e];
            const float mn = fmaxf(m[t], m1);
            const float a0 = __builtin_amdgcn_exp2f(m[t] - mn);
            const float a1 = __builtin_amdgcn_exp2f(m1 - mn);
            accl[t][0] = a0 * accl[t][0] + a1 * ml[t * 64 + lane_e];
#pragma unroll
            for (int x = 0; x < NVB; ++x)
                acc[t][x] = a0 * acc[t][x] + a1 * macc[(t * NVB + x) * 64 + lane_e];
        }
    }
    const auto ro = chunk_rsrc(out, int64_t(it.q0) * row_elems, 2, it.nq, H, D);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        // every row of accl holds the lane's query's sum
        const float inv = 1.f / accl[t][0];
        const uint32_t ooff = uint32_t((((trow_e + 16 * t) * H + h) * D + 4 * g_e) * 2);
#pragma unroll
        for (int x = 0; x < NVB; ++x)
            buf_store8(ro, ooff + x * 32,
                       u32x2{cvt_bf2(acc[t][x][0] * inv, acc[t][x][1] * inv),
                             cvt_bf2(acc[t][x][2] * inv, acc[t][x][3] * inv)});
    }
}

// Query tiles per wave and key parts per block, chosen by measurement on
// MI355X.
#ifndef LA_ATTN_QT_64
#define LA_ATTN_QT_64 2
#endif
#ifndef LA_ATTN_KH_64
#define LA_ATTN_KH_64 2
#endif
#ifndef LA_ATTN_QT_128
#define LA_ATTN_QT_128 2
#endif
#ifndef LA_ATTN_KH_128
#define LA_ATTN_KH_128 2
#endif

}  // namespace

extern "C" la_status la_attn_packed(const void* q, const void* k, const void* v, la_dtype dtype,
                                    int32_t H, int32_t d_k, int32_t d_v, float scale,
                                    const int32_t* items, int32_t n_items, int32_t n_tokens,
                                    const void* ext_k, const void* ext_v, int32_t n_ext_tokens,
                                    void* out, void* stream) {
    if (dtype != LA_BF16 && dtype != LA_F32) return LA_ERR_INVALID_ARG;
    if (dtype != LA_BF16) return LA_ERR_UNSUPPORTED;
    if (d_k != d_v || (d_k != 64 && d_k != 128)) return LA_ERR_UNSUPPORTED;
    if (H < 1 || n_items < 0 || n_tokens < 0 || n_ext_tokens < 0 || !std::isfinite(scale) ||
        !(scale > 0.f))
        return LA_ERR_INVALID_ARG;
    if (n_items == 0) return LA_OK;
    if (!q || !k || !v || !out || !items) return LA_ERR_INVALID_ARG;
    if (n_ext_tokens > 0 && (!ext_k || !ext_v)) return LA_ERR_INVALID_ARG;
    for (const void* p : {q, k, v, static_cast<const void*>(out)})
        if (reinterpret_cast<uintptr_t>(p) & 15u) return LA_ERR_INVALID_ARG;
    if ((ext_k && (reinterpret_cast<uintptr_t>(ext_k) & 15u)) ||
        (ext_v && (reinterpret_cast<uintptr_t>(ext_v) & 15u)))
        return LA_ERR_INVALID_ARG;
    if (int64_t(n_tokens) * H * d_k >= (int64_t(1) << 40) ||
        int64_t(n_ext_tokens) * H * d_k >= (int64_t(1) << 40) ||
        int64_t(kChunk) * H * d_k * 2 >= (int64_t(1) << 31) ||
        int64_t(n_items) * H * kThreads >= (int64_t(1) << 32))
        return LA_ERR_INVALID_ARG;
    const float scale_log2 = scale * 1.4426950408889634f;   // exp(x) = exp2(x log2 e)
    const auto* its = reinterpret_cast<const AttnItem*>(items);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(unsigned(int64_t(n_items) * H));
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kk = static_cast<const uint16_t*>(k);
    const auto* vv = static_cast<const uint16_t*>(v);
    const auto* ek = static_cast<const uint16_t*>(ext_k);
    const auto* ev = static_cast<const uint16_t*>(ext_v);
    auto* oo = static_cast<uint16_t*>(out);
    if (d_k == 64)
        hipLaunchKernelGGL((attn_kernel_bf16<64, LA_ATTN_QT_64, LA_ATTN_KH_64>), grid,
                           dim3(64 * LA_ATTN_KH_64 * (4 / LA_ATTN_QT_64)), 0, st, qq, kk, vv, ek,
                           ev, its, oo, H, scale_log2);
    else
        hipLaunchKernelGGL((attn_kernel_bf16<128, LA_ATTN_QT_128, LA_ATTN_KH_128>), grid,
                           dim3(64 * LA_ATTN_KH_128 * (4 / LA_ATTN_QT_128)), 0, st, qq, kk, vv, ek,
                           ev, its, oo, H, scale_log2);
    if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    return LA_OK;
}
