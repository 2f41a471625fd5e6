// Packed chunked causal linear-attention scan for gfx950 (MI355X).
//
// Source: "Serving 0.88M TPS from Two RTXs and Mac Minis", section "Kernels":
// linear attention is evaluated in 64-token chunks with a few 64x64 matrix
// products each (paragraph "Tensor cores for linear attention"), and one scan
// covers every view of a pass in three launches (paragraph "One scan per
// pass"); branches of all requests share the packed pass (paragraph "Shared
// branch passes") and start from their view's state (section "Long
// Requests").  Per head, with an fp32 state S of shape d x d:
//     S_t = S_{t-1} + k_t^T v_t,   o_t = q_t S_t.
// Chunked over a block of chunks c with S_in the state before the chunk:
//     O_c = Q_c S_in + tril(Q_c K_c^T) V_c,   S_in(next) = S_in + K_c^T V_c.
//
// The three launches:
//   delta_kernel   one workgroup per (delta block, head): sum over the block's
//                  chunks of K_c^T V_c, written to a workspace slot
//   prefix_kernel  one thread per (scanned segment, head, 1 or 4 state
//                  elements): inclusive prefix over the segment's slots, in
//                  place; the total of a view goes to final_state
//   output_kernel  one workgroup per (work block, head): chunk by chunk,
//                  O^T = S^T Q^T + V^T P^T with P = tril(Q K^T), carrying S in
//                  registers across the block's chunks
// For small passes the prefix launch is left out (the two-launch form): each
// output workgroup sums the slots before its block itself, in the same order.
//
// MFMA use (v_mfma_f32_16x16x32_bf16 for bf16, v_mfma_f32_16x16x4_f32 for
// fp32).  Accumulator layout of a 16x16 tile: lane l = 16 g + c holds rows
// 4 g + j (j = 0..3) of column c.  An A operand gives each lane one row
// (l % 16), a B operand one column (l % 16); the lane's group g = l / 16 and
// element index select k-slots.  The contraction sums over all k-slots, so
// any bijection from (g, element) to the contracted index is valid as long as
// A and B use the same one.  That freedom lets accumulator registers feed the
// next product directly: a tile's 4 rows 4g + j become the k-slots of lane
// group g, two row-tiles making the 8 bf16 elements of one K=32 step.
//
// Work split of launch 3 (bf16 path): NP workgroups share a (work block,
// head), each computing D / NP output features (NP = 1 at d = 64, 2 at
// d = 128; the parts of one item run on one XCD).  Inside a workgroup each
// wave owns 16 tokens of every chunk for the outputs and a few state tiles
// for the carry S += K^T V; each chunk the waves publish S^T as two bf16
// terms (hi + lo) in LDS for the inter-chunk product.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <type_traits>

#include "linattn.h"
#include "piece.h"
#include "tiles.h"

namespace {

// Work items (one per block or delta block and head) split over NP
// workgroups by output feature.  Workgroups go to the 8 XCDs round-robin by
// id, so the NP parts of one item get ids 8 apart: they run on one XCD at
// about the same time and their common q / k reads meet in its L2.
template <int NP>
__device__ __forceinline__ void split_id(int bid, int& item, int& part) {
    if constexpr (NP == 1) {
        item = bid;
        part = 0;
    } else {
        item = (bid / (8 * NP)) * 8 + bid % 8;
        part = (bid / 8) % NP;
    }
}
template <int NP>
inline int64_t split_grid(int64_t items) {
    return NP == 1 ? items : (items + 7) / 8 * 8 * NP;
}

// ---------------------------------------------------------------------------
// Plan descriptors (see linattn.h).
// ---------------------------------------------------------------------------
struct BlockDesc {
    int tok0, ntok, sin_slot, delta_slot, seed, seg, slot0, final_row;
};
struct DeltaDesc {
    int tok0, ntok, slot, seg;
};
struct ScanDesc {
    int first_slot, n_slots, final_row, seg;
};

// Every kernel first checks that the device plan is the one its la_pass_info
// describes (magic word and the planner's hash); on a mismatch it records
// LA_ERR_PLAN in the workspace header and does no work.
struct PlanCheck {
    const int32_t* plan;
    int* hdr;
    int hash;
    __device__ bool ok() const {
        if (plan[0] == LA_PLAN_MAGIC && plan[LA_PLAN_HASH_WORD] == hash) return true;
        if (threadIdx.x == 0)
            __hip_atomic_fetch_or(hdr + piece::kStatusWord, LA_ERR_PLAN, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
};

// ===========================================================================
// Launch 1: per delta block and head, sum over chunks of K_c^T V_c.  NP
// workgroups share a (delta block, head) item, each summing the state
// columns of D / NP value features (it reads all of K and its part of V).
// ===========================================================================
template <int D, int NP>
struct Delta1 {
    static constexpr int NW = 4;                       // waves per workgroup
    static constexpr int R = 4;                        // tokens per staging block
    static constexpr int DVW = D / NP;                 // value features per workgroup
    static constexpr int NKB = D / 16, NVB = DVW / 16;
    // a wave owns VBW column blocks x KBW row blocks of the state
    static constexpr int VBW = NVB >= NW ? NVB / NW : 1;
    static constexpr int KBW = NVB >= NW ? NKB : NKB * NVB / NW;
    static_assert(NVB % NW == 0 || NW % NVB == 0, "state tiles split evenly over the waves");
    __device__ static int vb0(int w) { return NVB >= NW ? w * VBW : w % NVB; }
    __device__ static int kb0(int w) { return NVB >= NW ? 0 : (w / NVB) * KBW; }
};

template <int D, int NP>
__global__ __launch_bounds__(kThreads) void delta_kernel_bf16(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const DeltaDesc* __restrict__ deltas, float* __restrict__ ws, int H, int n_items,
    PlanCheck pc) {
    if (!pc.ok()) return;
    using D1 = Delta1<D, NP>;
    constexpr int R = D1::R, DVW = D1::DVW, NKB = D1::NKB, NVB = D1::NVB;
    constexpr int VBW = D1::VBW, KBW = D1::KBW, DD = D * D;
    using ST = Stage<D, R>;
    constexpr int NPER = KVStage<D, DVW, R, kThreads>::NPER;
    constexpr int LDV = ST::template LDV<DVW>;
    __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * ST::LDR];   // K, row-major
    __shared__ __attribute__((aligned(16))) uint16_t sV[kChunk * LDV];       // V part, row-major

    int item, part;
    split_id<NP>(blockIdx.x, item, part);
    if (item >= n_items) return;   // whole workgroup: padding of the split grid
    const int h = item % H;
    const DeltaDesc dd = deltas[item / H];
    const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int vbw = D1::vb0(w), kbw = D1::kb0(w);

    f32x4 S[VBW][KBW];
#pragma unroll
    for (int x = 0; x < VBW; ++x)
#pragma unroll
        for (int i = 0; i < KBW; ++i) S[x][i] = zero4();

    const int nch = (dd.ntok + kChunk - 1) / kChunk;
    const int64_t row_elems = int64_t(H) * D;
    const int vcg0 = part * (DVW / 8);
    // two chunks in flight: registers A hold the even chunks, B the odd ones
    BlkR<R> pa[NPER], pb[NPER];
    auto load = [&](BlkR<R> (&dst)[NPER], int c) {
        const int64_t first = (int64_t(dd.tok0) + c * kChunk) * row_elems;
        const int rows = min(kChunk, dd.ntok - c * kChunk);   // <= 0: empty window
        load_kv<D, DVW, R, kThreads, NPER>(dst, chunk_rsrc(k, first, 2, rows, H, D),
                                           chunk_rsrc(v, first, 2, rows, H, D), vcg0, H, h);
    };
    auto stage = [&](const BlkR<R> (&cur)[NPER]) {
        stage_kv_rows<D, DVW, R, kThreads, NPER>(cur, sK, sV);
    };
    // S += K^T V of the chunk staged in LDS
    auto accumulate = [&]() {
#pragma unroll
        for (int ks = 0; ks < kChunk / 32; ++ks) {
#pragma unroll
            for (int x = 0; x < VBW; ++x) {
                const int vb = vbw + x;
                const u32x4 bv = tr_frag(sV, LDV, vb * 16, ks, g, c16);
#pragma unroll
                for (int i = 0; i < KBW; ++i) {
                    const int kb = kbw + i;
                    const u32x4 ak = tr_frag(sK, ST::LDR, kb * 16, ks, g, c16);
                    S[x][i] = mfma_bf16(ak, bv, S[x][i]);
                }
            }
        }
    };
    // The loop is rotated like launch 3's: a chunk is staged at the end of
    // the previous step, when exactly one later chunk's loads were issued
    // after its own, and the loop entry has the same outstanding loads as the
    // back edge (chunk 1 in B).  The wait before each staging then leaves the
    // next chunk in flight.  Loads past the last chunk read an empty window.
    load(pa, 0);
    __builtin_amdgcn_sched_barrier(0);   // keep chunk 0's loads ahead of chunk 1's
    load(pb, 1);
    stage(pa);
    for (int c = 0; c < nch; c += 2) {
        __syncthreads();
        load(pa, c + 2);
        accumulate();
        __syncthreads();
        if (c + 1 >= nch) break;
        stage(pb);
        __syncthreads();
        load(pb, c + 3);
        accumulate();
        __syncthreads();
        if (c + 2 >= nch) break;
        stage(pa);
    }
    // the block state streams to memory (nontemporal): the next launch reads
    // it once, and the stores then leave no dirty lines for the write-back at
    // the end of the kernel (launch 1 at the 272k-token pass: 709 -> 686 us)
    f32x4* dst = reinterpret_cast<f32x4*>(ws + ((int64_t)dd.slot * H + h) * DD);
#pragma unroll
    for (int x = 0; x < VBW; ++x)
#pragma unroll
        for (int i = 0; i < KBW; ++i)
            __builtin_nontemporal_store(S[x][i], &dst[((part * NVB + vbw + x) * NKB + kbw + i) * 64 + lane]);
}

// fp32 tiles: row-major [64][D+4] floats in LDS, loaded as 16-byte pieces.
template <int D>
struct F32Tiles {
    static constexpr int LD = D + 4;
    static constexpr int PIECES = kChunk * D / 4;      // 16-byte pieces per tile
    static constexpr int PER = PIECES / kThreads;       // per thread per tile
};

template <int D>
__device__ __forceinline__ void load_f32_tile(f32x4* regs, const float* __restrict__ base,
                                              int64_t tok0, int rows, int H, int h) {
    using TL = F32Tiles<D>;
    constexpr int PPR = D / 4;   // pieces per row
#pragma unroll
    for (int i = 0; i < TL::PER; ++i) {
        const int p = threadIdx.x + i * kThreads;
        const int row = p / PPR, col = (p % PPR) * 4;
        if (row < rows)
            regs[i] = *reinterpret_cast<const f32x4*>(base + ((tok0 + row) * H + h) * (int64_t)D + col);
        else
            regs[i] = zero4();
    }
}

template <int D>
__device__ __forceinline__ void store_f32_tile(float* dst, const f32x4* regs) {
    using TL = F32Tiles<D>;
    constexpr int PPR = D / 4;
#pragma unroll
    for (int i = 0; i < TL::PER; ++i) {
        const int p = threadIdx.x + i * kThreads;
        const int row = p / PPR, col = (p % PPR) * 4;
        *reinterpret_cast<f32x4*>(dst + row * TL::LD + col) = regs[i];
    }
}

// S[x][kb] += K^T V over one chunk, fp32 operands from row-major tiles.
template <int D>
__device__ __forceinline__ void f32_state_update(f32x4 (&S)[D / 64][D / 16], const float* sK,
                                                 const float* sV, int w, int g, int c16) {
    using TL = F32Tiles<D>;
    constexpr int NKB = D / 16, VBW = D / 64;
#pragma unroll 4
    for (int ks = 0; ks < kChunk / 4; ++ks) {
        const int u = ks * 4 + g;
#pragma unroll
        for (int x = 0; x < VBW; ++x) {
            const float bv = sV[u * TL::LD + (w * VBW + x) * 16 + c16];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                S[x][kb] = mfma_f32(sK[u * TL::LD + kb * 16 + c16], bv, S[x][kb]);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void delta_kernel_f32(
    const float* __restrict__ k, const float* __restrict__ v,
    const DeltaDesc* __restrict__ deltas, float* __restrict__ ws, int H, PlanCheck pc) {
    if (!pc.ok()) return;
    using TL = F32Tiles<D>;
    constexpr int NKB = D / 16, VBW = D / 64, DD = D * D;
    __shared__ __attribute__((aligned(16))) float sK[kChunk * TL::LD];
    __shared__ __attribute__((aligned(16))) float sV[kChunk * TL::LD];

    const int h = blockIdx.x % H;
    const DeltaDesc dd = deltas[blockIdx.x / H];
    const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, g = lane >> 4, c16 = lane & 15;

    f32x4 S[VBW][NKB];
#pragma unroll
    for (int x = 0; x < VBW; ++x)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) S[x][kb] = zero4();

    const int nch = (dd.ntok + kChunk - 1) / kChunk;
    f32x4 pk[TL::PER], pv[TL::PER];
    load_f32_tile<D>(pk, k, dd.tok0, min(kChunk, dd.ntok), H, h);
    load_f32_tile<D>(pv, v, dd.tok0, min(kChunk, dd.ntok), H, h);
    for (int c = 0; c < nch; ++c) {
        store_f32_tile<D>(sK, pk);
        store_f32_tile<D>(sV, pv);
        __syncthreads();
        if (c + 1 < nch) {
            const int64_t t0 = (int64_t)dd.tok0 + (c + 1) * kChunk;
            const int rows = min(kChunk, dd.ntok - (c + 1) * kChunk);
            load_f32_tile<D>(pk, k, t0, rows, H, h);
            load_f32_tile<D>(pv, v, t0, rows, H, h);
        }
        f32_state_update<D>(S, sK, sV, w, g, c16);
        __syncthreads();
    }
    f32x4* dst = reinterpret_cast<f32x4*>(ws + ((int64_t)dd.slot * H + h) * DD);
#pragma unroll
    for (int x = 0; x < VBW; ++x)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) dst[((w * VBW + x) * NKB + kb) * 64 + lane] = S[x][kb];
}

// ===========================================================================
// Launch 2: segmented inclusive prefix over each scanned segment's slots.
// One thread per EPT consecutive state elements of one (segment, head);
// consecutive threads take consecutive elements, so every slot access is a
// coalesced row.  Up to BATCH slot loads per thread are in flight at once
// (one memory round trip for segments of up to that many slots).  Slot
// j >= 1 is rewritten with the sum of slots 0..j; for a view that sum at
// the last slot is its final state, which also goes to final_state
// (row-major); branch blocks read their seed from the slot, whose lane
// layout gives 16-byte loads.
// Every element is summed from zero in slot order, whatever EPT.
// EPT = 1 with BATCH = 32 suits passes with few segments (one round trip for
// the long views, as many workgroups as elements allow); EPT = 4 with
// BATCH = 8 suits passes with many segment-heads, where one element per
// thread made tens of thousands of latency-bound workgroups (the 272k-token
// pass at d = 128: 65,536 of them).
// ===========================================================================
constexpr int64_t kPrefixWideGroups = 8192;   // workgroups at one element per thread

template <int D, int EPT, int BATCH, bool REWRITE_FIRST = false>
__global__ __launch_bounds__(kThreads) void prefix_kernel(const ScanDesc* __restrict__ scans,
                                                          float* __restrict__ ws,
                                                          float* __restrict__ final_state,
                                                          int H, PlanCheck pc) {
    if (!pc.ok()) return;
    static_assert(EPT == 1 || EPT == 4, "one element or one 16-byte piece per thread");
    using V = typename std::conditional<EPT == 4, f32x4, float>::type;
    constexpr int DD = D * D, WPS = DD / (kThreads * EPT);
    const int per_seg = H * WPS;
    const ScanDesc sd = scans[blockIdx.x / per_seg];
    const int rem = blockIdx.x % per_seg;
    const int h = rem / WPS;
    const int e = ((rem % WPS) * kThreads + threadIdx.x) * EPT;
    const int64_t stride = (int64_t)H * DD / EPT;   // one slot, in units of V
    V* p = reinterpret_cast<V*>(ws + ((int64_t)sd.first_slot * H + h) * DD + e);
    const int n = sd.n_slots;
    const int last_store = n;   // exclusive bound: a view's last slot gets its total too
    V acc = V(0.f);
    for (int j0 = 0; j0 < n; j0 += BATCH) {
        V x[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
            x[i] = (j0 + i < n) ? p[(j0 + i) * stride] : V(0.f);
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int j = j0 + i;
            acc += x[i];
            if ((REWRITE_FIRST || j >= 1) && j < last_store) p[j * stride] = acc;
        }
    }
    if (sd.final_row >= 0) {
        float* dst = final_state + ((int64_t)sd.final_row * H + h) * DD;
#pragma unroll
        for (int t = 0; t < EPT; ++t) {
            int row, col;
            slot_to_rc<D>(e + t, row, col);
            if constexpr (EPT == 4)
                dst[row * D + col] = acc[t];
            else
                dst[row * D + col] = acc;
        }
    }
}

// ===========================================================================
// Launch 3: outputs.  Per work block and head, chunk by chunk.
// ===========================================================================

// Initial state of a block, for the state tiles a lane carries: tile i is
// tile index tix[i] = vb * NKB + kb of the slot layout, and the lane holds
// S[kb*16 + 4g + j][vb*16 + c] (lane = 16 g + c), j = 0..3.
//   S_in = seed + own
// seed: zero (a view), the view's final state (a branch) or an external state
// (a shard branch); own: the segment-local sum of the earlier blocks' states.
// Three-launch form: the prefix launch has left own in slot sin_slot and each
// view's total in the view's last slot.  Two-launch form (`fused`): the slots hold the
// blocks' own states and the block sums them here, in slot order: own =
// slots slot0 .. sin_slot, a branch's seed = all slots of its view (scan
// entry `seed`); a view's last block also writes the view's total, own plus
// its own slot, to final_state.  Both forms add in the same order as the
// prefix launch (from zero, one slot after the other), so they give the same
// bits, and a branch's seed equals the final_state written for its view.
// B slots of loads in flight per batch (B * NT 16-byte pieces per lane).
template <int D, int NT, int B>
__device__ __forceinline__ void sum_slots(f32x4 (&acc)[NT], const int (&tix)[NT],
                                          const float* __restrict__ ws, int first, int n, int H,
                                          int h, int lane) {
    constexpr int64_t SLOT4 = D * D / 4;   // 16-byte pieces per slot
    const int64_t stride = int64_t(H) * SLOT4;
    const f32x4* p = reinterpret_cast<const f32x4*>(ws) + (int64_t(first) * H + h) * SLOT4 + lane;
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = zero4();
    int s = 0;
    for (; s + B <= n; s += B) {
        f32x4 x[B][NT];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int i = 0; i < NT; ++i) x[b][i] = p[(s + b) * stride + tix[i] * 64];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int i = 0; i < NT; ++i) acc[i] += x[b][i];
    }
    for (; s < n; ++s)
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[i] += p[s * stride + tix[i] * 64];
}

// The slot sums of the two-launch form keep B slots of loads in flight: 16
// pieces per lane (the register count of the kernels stays that of the
// three-launch form) or, where the kernel has registers to spare, 32.
template <int D, int NT, bool FUSED, int B = (NT >= 16 ? 1 : 16 / NT)>
__device__ __forceinline__ void block_init_state(
    f32x4 (&S)[NT], const int (&tix)[NT], const BlockDesc& bd, const ScanDesc* __restrict__ scans,
    const float* __restrict__ ws, float* __restrict__ final_state,
    const float* __restrict__ ext_state, int H, int h, int lane) {
    constexpr bool fused = FUSED;
    constexpr int NKB = D / 16, DD = D * D;
    const int g = lane >> 4, c16 = lane & 15;
    // row-major [D][D] seed (final_state or ext_state row) into the tiles
    auto read_rows = [&](const float* __restrict__ src) {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int kb = tix[i] % NKB, vb = tix[i] / NKB;
#pragma unroll
            for (int j = 0; j < 4; ++j) S[i][j] = src[(kb * 16 + 4 * g + j) * D + vb * 16 + c16];
        }
    };
#pragma unroll
    for (int i = 0; i < NT; ++i) S[i] = zero4();
    if (bd.seed <= -2) {
        read_rows(ext_state + ((int64_t)(-bd.seed - 2) * H + h) * DD);
    } else if (bd.seed >= 0) {
        if constexpr (fused) {
            const ScanDesc sc = scans[bd.seed];
            sum_slots<D, NT, B>(S, tix, ws, sc.first_slot, sc.n_slots, H, h, lane);
        } else {
            // the prefix launch left the view's total in its last slot too
            // (the same bits as its final_state row), in the lane layout
            const ScanDesc sc = scans[bd.seed];
            const f32x4* p = reinterpret_cast<const f32x4*>(
                ws + ((int64_t)(sc.first_slot + sc.n_slots - 1) * H + h) * DD);
#pragma unroll
            for (int i = 0; i < NT; ++i) S[i] = p[tix[i] * 64 + lane];
        }
    }
    if (bd.sin_slot >= 0) {
        f32x4 own[NT];
        if constexpr (fused) {
            sum_slots<D, NT, B>(own, tix, ws, bd.slot0, bd.sin_slot - bd.slot0 + 1, H, h, lane);
        } else {
            const f32x4* p = reinterpret_cast<const f32x4*>(ws + ((int64_t)bd.sin_slot * H + h) * DD);
#pragma unroll
            for (int i = 0; i < NT; ++i) own[i] = p[tix[i] * 64 + lane];
        }
#pragma unroll
        for (int i = 0; i < NT; ++i) S[i] += own[i];
    }
    if (fused && bd.final_row >= 0) {
        const f32x4* p = reinterpret_cast<const f32x4*>(ws + ((int64_t)bd.delta_slot * H + h) * DD);
        float* dst = final_state + ((int64_t)bd.final_row * H + h) * DD;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const f32x4 t = S[i] + p[tix[i] * 64 + lane];
            const int kb = tix[i] % NKB, vb = tix[i] / NKB;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[(kb * 16 + 4 * g + j) * D + vb * 16 + c16] = t[j];
        }
    }
}

// Launch 3 (bf16): NP workgroups share a (work block, head) item, each
// computing the DV = D / NP output features starting at part * DV and
// carrying the matching state columns.  NW waves per workgroup: wave
// w = 4 hv + tb computes the outputs of tokens tb*16 .. tb*16+15 for VBH
// feature tiles (feature part hv of the workgroup's DV features), and owns
// TPW state tiles (vb_own, kb0 .. kb0+TPW-1; vb_own local to the part) for
// the carry.
template <int D, int NP, int NW_>
struct Out3 {
    static constexpr int NP_ = NP, NW = NW_;
    static constexpr int NT = 64 * NW;
    static constexpr int R = 4;                       // tokens per staging block
    static constexpr int DV = D / NP;                 // output features per workgroup
    static constexpr int NKB = D / 16, NVB = DV / 16, NKS = D / 32;
    static constexpr int NHV = NW / 4;                // feature parts per workgroup
    static constexpr int VBH = NVB / NHV;             // output tiles per wave
    static constexpr int TPW = NVB * NKB / NW;        // carry tiles per wave
    static_assert(NW % 4 == 0 && NVB % NHV == 0, "waves cover 4 token blocks x feature parts");
    static_assert(NW % NVB == 0 && NKB % TPW == 0,
                  "a wave's carry tiles share one state column block");
    __device__ static int vb_own(int w) { return w % NVB; }
    __device__ static int kb0(int w) { return (w / NVB) * TPW; }
};

// Launch configurations, chosen by measurement on MI355X: launch 1 splits
// each item over DELTA_NP workgroups, launch 3 over OUT_NP workgroups of
// OUT_NW waves (the split-precision launch 3 over SPLIT_NP of SPLIT_NW).  At
// d = 128 one workgroup of 8 waves per item (both 64-feature halves, q and k
// read once) ran launch 3 of the 272k-token pass in 2505 us against 2345 us
// for two workgroups of 4 waves (one per half): the larger workgroup needs
// 105 KB of LDS, one per CU.
#ifndef LA_DELTA_NP_64
#define LA_DELTA_NP_64 1
#endif
#ifndef LA_DELTA_NP_128
#define LA_DELTA_NP_128 1
#endif
#ifndef LA_OUT_NP_64
#define LA_OUT_NP_64 1
#endif
#ifndef LA_OUT_NW_64
#define LA_OUT_NW_64 4
#endif
#ifndef LA_OUT_NP_128
#define LA_OUT_NP_128 2
#endif
#ifndef LA_OUT_NW_128
#define LA_OUT_NW_128 4
#endif
#ifndef LA_SPLIT_NP_128
#define LA_SPLIT_NP_128 2
#endif
#ifndef LA_SPLIT_NW_128
#define LA_SPLIT_NW_128 4
#endif
template <int D>
struct LaunchCfg;
template <>
struct LaunchCfg<64> {
    static constexpr int DELTA_NP = LA_DELTA_NP_64;
    using O3 = Out3<64, LA_OUT_NP_64, LA_OUT_NW_64>;
    using O3S = O3;   // split-precision launch 3
};
template <>
struct LaunchCfg<128> {
    static constexpr int DELTA_NP = LA_DELTA_NP_128;
    using O3 = Out3<128, LA_OUT_NP_128, LA_OUT_NW_128>;
    using O3S = Out3<128, LA_SPLIT_NP_128, LA_SPLIT_NW_128>;
};

// Output feature order of the bf16 output launch (64 output features per
// workgroup, 4 output tiles per wave): row 4 g + j of output tile x holds
// feature 32 (x >> 1) + 8 g + 4 (x & 1) + j, so lane group g ends with
// features 8 g .. 8 g + 7 (tiles 0, 1) and 32 + 8 g .. 32 + 8 g + 7 (tiles
// 2, 3) of its token: two 16-byte stores, and the four lane groups of a token
// cover 64 contiguous bytes of its row per store.  The A operands follow:
// V^T rows are read in that order, and S^T is published at LDS row
// out_row(f), which puts the feature that A-operand lane c of tile x needs at
// row 16 x + c.
__device__ __forceinline__ int out_row(int f) {
    return 32 * (f >> 5) + 16 * ((f >> 2) & 1) + 4 * ((f >> 3) & 3) + (f & 3);
}

// LDS rows of the bf16 output launch's K and S^T tiles.  d = 64: the common
// 160-byte rows with the scol swizzle.  d = 128: 288-byte rows, and rows with
// bit 4 set keep the two 8-element halves of each 16-element group swapped;
// in a 64-bank model this leaves no bank conflicts in the 8-byte S^T
// publication stores (their 16 lanes hit rows r and r + 16), the 16-byte
// S^T and K fragment reads, the transposed K reads of the carry and the K
// staging stores (272-byte rows without the swizzle: two-way conflicts in
// the publication and the transposed reads).
template <int D>
struct OutLds {
    static constexpr int LDR = D == 128 ? D + 16 : Stage<D, 4>::LDR;
    __device__ static int col(int row, int k) {
        if constexpr (D == 128) return k ^ ((row & 16) >> 1);
        return scol<D>(row, k);
    }
};

// The outputs of one wave for one chunk: its 16 tokens (token block TB), the
// 64 output features of feature half hv of the workgroup in the order above.  Specialised per
// TB so that the causal structure (TB + 1 score tiles, TB / 2 + 1
// intra-chunk steps) is known at compile time and every loop runs over
// independent accumulators with its LDS fragments loaded in batches.
template <int D, int TB, int VBH, int LDV>
__device__ __forceinline__ void out_tiles(const uint16_t* sK, const uint16_t* sV,
                                          const uint16_t* sSh, const uint16_t* sSl,
                                          const u32x4 (&qf)[D / 32], int hv, int g, int c16,
                                          f32x4 (&acc)[VBH]) {
    static_assert(VBH == 4, "one wave covers the 64 output features of its workgroup");
    constexpr int NKS = D / 32;
    constexpr int LDR = OutLds<D>::LDR;
    // P^T tiles (ub, TB), ub <= TB: P^T[u][t] = sum_d K[u][d] Q[t][d]
    f32x4 p[TB + 1];
#pragma unroll
    for (int ub = 0; ub <= TB; ++ub) p[ub] = zero4();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        u32x4 kf[TB + 1];
#pragma unroll
        for (int ub = 0; ub <= TB; ++ub)
            kf[ub] = lds_u32x4(sK + (ub * 16 + c16) * LDR + ks * 32 + 8 * g);
#pragma unroll
        for (int ub = 0; ub <= TB; ++ub) p[ub] = mfma_bf16(kf[ub], qf[ks], p[ub]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)   // causal mask inside the diagonal tile: u <= t
        if (4 * g + j > c16) p[TB][j] = 0.f;
    u32x2 pb[4];
#pragma unroll
    for (int ub = 0; ub < 4; ++ub)
        pb[ub] = ub <= TB ? u32x2{cvt_bf2(p[ub][0], p[ub][1]), cvt_bf2(p[ub][2], p[ub][3])}
                          : u32x2{0u, 0u};

    // inter-chunk: O^T += S_hi^T Q^T + S_lo^T Q^T
#pragma unroll
    for (int x = 0; x < VBH; ++x) acc[x] = zero4();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        u32x4 ah[VBH], al[VBH];
#pragma unroll
        for (int x = 0; x < VBH; ++x) {
            const int row = hv * 64 + x * 16 + c16;
            const int o = row * LDR + OutLds<D>::col(row, ks * 32 + 8 * g);
            ah[x] = lds_u32x4(sSh + o);
            al[x] = lds_u32x4(sSl + o);
        }
#pragma unroll
        for (int x = 0; x < VBH; ++x) acc[x] = mfma_bf16(ah[x], qf[ks], acc[x]);
#pragma unroll
        for (int x = 0; x < VBH; ++x) acc[x] = mfma_bf16(al[x], qf[ks], acc[x]);
    }
    // intra-chunk: O^T += V^T P^T, k-slots (g, i) -> u = ub_{i/4}*16 + 4g + i%4
#pragma unroll
    for (int pp = 0; pp <= TB / 2; ++pp) {
        const u32x4 bp = cat2(pb[2 * pp], pb[2 * pp + 1]);
        u32x4 av[VBH];
#pragma unroll
        for (int x = 0; x < VBH; ++x) {
            // as tr_frag, with lane c of the tile receiving feature
            // 32 (x >> 1) + 8 (c >> 2) + 4 (x & 1) + (c & 3)
            const uint16_t* pv = sV + (4 * g + (c16 >> 2)) * LDV + hv * 64 + 32 * (x >> 1) +
                                 8 * (c16 & 3) + 4 * (x & 1);
            av[x] = cat2(lds_tr4(pv + (2 * pp) * 16 * LDV), lds_tr4(pv + (2 * pp + 1) * 16 * LDV));
        }
#pragma unroll
        for (int x = 0; x < VBH; ++x) acc[x] = mfma_bf16(av[x], bp, acc[x]);
    }
}

template <int D, class O3, bool FUSED>
__global__ __launch_bounds__(O3::NT) void output_kernel_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const BlockDesc* __restrict__ blocks,
    const ScanDesc* __restrict__ scans, const float* __restrict__ ws,
    float* __restrict__ final_state, const float* __restrict__ ext_state,
    uint16_t* __restrict__ out, int H, int n_items, PlanCheck pc) {
    if (!pc.ok()) return;
    constexpr int R = O3::R, NT = O3::NT, NP = O3::NP_, DV = O3::DV;
    constexpr int NKB = O3::NKB, NVB = O3::NVB, NKS = O3::NKS, VBH = O3::VBH, TPW = O3::TPW;
    constexpr int NPER = KVStage<D, DV, R, NT>::NPER;
    constexpr int LDR = OutLds<D>::LDR;
    // V rows of 192 bytes: the permuted V^T fragment reads of out_tiles (8-byte
    // pieces 16 bytes apart on four rows) and the carry's reads both hit every
    // LDS bank at most once per 128 bytes
    constexpr int LDV = DV + 32;
    static_assert(DV == 64 * O3::NHV && VBH == 4, "waves cover 64-feature halves");
    __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * LDR];   // K, row-major
    __shared__ __attribute__((aligned(16))) uint16_t sV[kChunk * LDV];   // V part, row-major
    __shared__ __attribute__((aligned(16))) uint16_t sSh[DV * LDR];   // S^T, bf16 high term
    __shared__ __attribute__((aligned(16))) uint16_t sSl[DV * LDR];   // S^T, bf16 low term

    int item, part;
    split_id<NP>(blockIdx.x, item, part);
    if (item >= n_items) return;   // whole workgroup: padding of the split grid
    const int h = item % H;
    const BlockDesc bd = blocks[item / H];
    const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int tb = w & 3, hv = O3::NHV == 1 ? 0 : w >> 2;
    const int vbo = O3::vb_own(w), kbo = O3::kb0(w);   // vbo local to the part
    const int vbg = part * NVB + vbo;                   // global column block

    const int nch = (bd.ntok + kChunk - 1) / kChunk;
    const int64_t row_elems = int64_t(H) * D;
    // this lane's token within the chunk and the byte offsets of its q / out
    // row pieces inside a chunk window
    const int trow = tb * 16 + c16;
    const uint32_t qoff = uint32_t(((trow * H + h) * D + 8 * g) * 2);
    const uint32_t ooff = uint32_t(((trow * H + h) * D + part * DV + hv * 64 + 8 * g) * 2);
    const int vcg0 = part * (DV / 8);

    // one chunk in flight: kv / qn hold chunk c + 1 while chunk c is computed
    BlkR<R> kv[NPER];
    u32x4 qf[NKS], qn[NKS];
    auto load = [&](int c, u32x4 (&qdst)[NKS]) {
        const int64_t first = (int64_t(bd.tok0) + c * kChunk) * row_elems;
        const int rows = min(kChunk, bd.ntok - c * kChunk);   // <= 0: empty window
        load_kv<D, DV, R, NT, NPER>(kv, chunk_rsrc(k, first, 2, rows, H, D),
                                    chunk_rsrc(v, first, 2, rows, H, D), vcg0, H, h);
        const auto rq = chunk_rsrc(q, first, 2, rows, H, D);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qdst[ks] = buf_load16(rq, qoff + ks * 64);
    };
    // the first chunk's loads go out before the initial state is read; q goes
    // straight to the registers the products read (later chunks' q lands in
    // qn while the current chunk is computed)
    load(0, qf);

    // carry state: tiles (vbg, kbo + i); lane holds S[kb*16 + 4g + j][vbg*16 + c16]
    f32x4 S[TPW];
    {
        int tix[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) tix[i] = vbg * NKB + kbo + i;
        // at d = 64 the two-launch kernel has registers for 8 slots in flight
        block_init_state<D, TPW, FUSED, (FUSED && D == 64 ? 8 : 16 / TPW)>(
            S, tix, bd, scans, ws, final_state, ext_state, H, h, lane);
    }

    // LDS inputs of one chunk: S^T = S_hi + S_lo (bf16 terms) for the
    // inter-chunk product (lane holds 4 consecutive d_k of row vbo*16 + c16
    // of the part's S^T), K row-major and transposed, V transposed.
    auto publish_and_stage = [&]() {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const f32x4 s = S[i];
            const uint32_t h01 = cvt_bf2(s[0], s[1]), h23 = cvt_bf2(s[2], s[3]);
            const uint32_t l01 = cvt_bf2(s[0] - bf_lo(h01), s[1] - bf_hi(h01));
            const uint32_t l23 = cvt_bf2(s[2] - bf_lo(h23), s[3] - bf_hi(h23));
            const int f = vbo * 16 + c16;   // feature within the part
            const int row = (f & ~63) + out_row(f & 63);
            const int off = row * LDR + OutLds<D>::col(row, (kbo + i) * 16 + 4 * g);
            *reinterpret_cast<u32x2*>(sSh + off) = u32x2{h01, h23};
            *reinterpret_cast<u32x2*>(sSl + off) = u32x2{l01, l23};
        }
        stage_kv_rows<D, DV, R, NT, NPER, LDV, LDR>(kv, sK, sV);
    };
    // The loop is rotated: chunk c + 1 is staged (and its q moved to qf) at
    // the end of iteration c, right after chunk c's output stores.  Its loads
    // were issued before those stores, so the waits for them leave the
    // stores in flight; the loop entry has no loads outstanding, so nothing
    // merges into a wait for the stores either.
    publish_and_stage();
    // every load of the entry is complete here (chunk 0's q is needed first
    // thing anyway); stating it lets the wait counts inside the loop be exact
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    for (int c = 0; c < nch; ++c) {
        __syncthreads();
        // fetch the next chunk (an empty window past the last one)
        load(c + 1, qn);

        const int rows = min(kChunk, bd.ntok - c * kChunk);
        const int64_t first = (int64_t(bd.tok0) + c * kChunk) * row_elems;

        // O^T tiles: this wave's 16 tokens, the 64 output features of half hv
        f32x4 acc[VBH];
        switch (tb) {
            case 0: out_tiles<D, 0, VBH, LDV>(sK, sV, sSh, sSl, qf, hv, g, c16, acc); break;
            case 1: out_tiles<D, 1, VBH, LDV>(sK, sV, sSh, sSl, qf, hv, g, c16, acc); break;
            case 2: out_tiles<D, 2, VBH, LDV>(sK, sV, sSh, sSl, qf, hv, g, c16, acc); break;
            default: out_tiles<D, 3, VBH, LDV>(sK, sV, sSh, sSl, qf, hv, g, c16, acc); break;
        }
        // lane holds O[t = tb*16 + c16][part*DV + hv*64 + 32 (x >> 1) + 8g + 4 (x & 1) + j]:
        // piece A (features 8g ..) and piece B (32 + 8g ..) of its token.  Lanes
        // of neighbouring tokens (c16, c16 ^ 1) swap one piece, so that each of
        // the two stores writes whole 128-byte feature rows (one token each from
        // 8 lanes): the even token's row in the first, the odd token's in the
        // second.
        {
            const auto ro = chunk_rsrc(out, first, 2, rows, H, D);
            u32x4 pc[2];
#pragma unroll
            for (int y = 0; y < 2; ++y)
                pc[y] = u32x4{cvt_bf2(acc[2 * y][0], acc[2 * y][1]),
                              cvt_bf2(acc[2 * y][2], acc[2 * y][3]),
                              cvt_bf2(acc[2 * y + 1][0], acc[2 * y + 1][1]),
                              cvt_bf2(acc[2 * y + 1][2], acc[2 * y + 1][3])};
            const bool odd = (c16 & 1) != 0;
            const u32x4 give = odd ? pc[0] : pc[1];
            u32x4 got;
#pragma unroll
            for (int i = 0; i < 4; ++i)   // quad_perm [1, 0, 3, 2]: lane c16 ^ 1
                got[i] = __builtin_amdgcn_mov_dpp(int(give[i]), 0xB1, 0xF, 0xF, false);
            const uint32_t row_bytes = uint32_t(H * D * 2);
            buf_store16u(ro, odd ? ooff - row_bytes + 64 : ooff, odd ? got : pc[0]);
            buf_store16u(ro, odd ? ooff + 64 : ooff + row_bytes, odd ? pc[1] : got);
        }
        if (c + 1 >= nch) break;   // no carry and no staging after the last chunk
        // carry: S += K^T V for this wave's tiles
#pragma unroll
        for (int ks = 0; ks < kChunk / 32; ++ks) {
            const u32x4 bv = tr_frag(sV, LDV, vbo * 16, ks, g, c16);
#pragma unroll
            for (int i = 0; i < TPW; ++i)
                S[i] = mfma_bf16(tr_frag(sK, LDR, (kbo + i) * 16, ks, g, c16), bv, S[i]);
        }
        __syncthreads();
        publish_and_stage();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = qn[ks];
    }
}

template <int D, bool FUSED>
__global__ __launch_bounds__(kThreads) void output_kernel_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const BlockDesc* __restrict__ blocks, const ScanDesc* __restrict__ scans,
    const float* __restrict__ ws, float* __restrict__ final_state,
    const float* __restrict__ ext_state, float* __restrict__ out, int H, PlanCheck pc) {
    if (!pc.ok()) return;
    using TL = F32Tiles<D>;
    constexpr int NKB = D / 16, VBW = D / 64;
    __shared__ __attribute__((aligned(16))) float sQ[kChunk * TL::LD];
    __shared__ __attribute__((aligned(16))) float sK[kChunk * TL::LD];
    __shared__ __attribute__((aligned(16))) float sV[kChunk * TL::LD];

    const int h = blockIdx.x % H;
    const BlockDesc bd = blocks[blockIdx.x / H];
    const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, g = lane >> 4, c16 = lane & 15;

    f32x4 S[VBW][NKB];
    {
        // the wave's tiles (w * VBW + x, kb), flattened as x * NKB + kb
        int tix[VBW * NKB];
#pragma unroll
        for (int x = 0; x < VBW; ++x)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) tix[x * NKB + kb] = (w * VBW + x) * NKB + kb;
        f32x4 Sf[VBW * NKB];
        block_init_state<D, VBW * NKB, FUSED>(Sf, tix, bd, scans, ws, final_state, ext_state,
                                              H, h, lane);
#pragma unroll
        for (int x = 0; x < VBW; ++x)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) S[x][kb] = Sf[x * NKB + kb];
    }

    const int nch = (bd.ntok + kChunk - 1) / kChunk;
    f32x4 pq[TL::PER], pk[TL::PER], pv[TL::PER];
    {
        const int rows = min(kChunk, bd.ntok);
        load_f32_tile<D>(pq, q, bd.tok0, rows, H, h);
        load_f32_tile<D>(pk, k, bd.tok0, rows, H, h);
        load_f32_tile<D>(pv, v, bd.tok0, rows, H, h);
    }
    for (int c = 0; c < nch; ++c) {
        store_f32_tile<D>(sQ, pq);
        store_f32_tile<D>(sK, pk);
        store_f32_tile<D>(sV, pv);
        __syncthreads();
        if (c + 1 < nch) {
            const int64_t tn = (int64_t)bd.tok0 + (c + 1) * kChunk;
            const int rn = min(kChunk, bd.ntok - (c + 1) * kChunk);
            load_f32_tile<D>(pq, q, tn, rn, H, h);
            load_f32_tile<D>(pk, k, tn, rn, H, h);
            load_f32_tile<D>(pv, v, tn, rn, H, h);
        }
        const int rows = min(kChunk, bd.ntok - c * kChunk);
        const int64_t t0 = (int64_t)bd.tok0 + c * kChunk;
#pragma unroll 1
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 p[4];
#pragma unroll
            for (int ub = 0; ub < 4; ++ub) {
                p[ub] = zero4();
                if (ub > tb) continue;
#pragma unroll 4
                for (int ks = 0; ks < D / 4; ++ks)
                    p[ub] = mfma_f32(sK[(ub * 16 + c16) * TL::LD + ks * 4 + g],
                                     sQ[(tb * 16 + c16) * TL::LD + ks * 4 + g], p[ub]);
                if (ub == tb) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (4 * g + j > c16) p[ub][j] = 0.f;
                }
            }
            const int trow = tb * 16 + c16;
#pragma unroll
            for (int x = 0; x < VBW; ++x) {
                const int vb = w * VBW + x;
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc = mfma_f32(S[x][kb][j], sQ[trow * TL::LD + kb * 16 + 4 * g + j], acc);
#pragma unroll
                for (int ub = 0; ub < 4; ++ub) {
                    if (ub > tb) continue;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc = mfma_f32(sV[(ub * 16 + 4 * g + j) * TL::LD + vb * 16 + c16],
                                       p[ub][j], acc);
                }
                if (trow < rows) {
                    float* o = out + ((t0 + trow) * H + h) * (int64_t)D + vb * 16 + 4 * g;
                    *reinterpret_cast<f32x4*>(o) = acc;
                }
            }
        }
        if (c + 1 < nch) f32_state_update<D>(S, sK, sV, w, g, c16);
        __syncthreads();
    }
}

// ===========================================================================
// Split-precision fp32 path (section "Kernels", paragraph "Tensor cores for
// linear attention": the page runs its fp32 data on tf32 tensor cores with
// each product split into three for accuracy).  Here each fp32 operand x is
// split into two bf16 terms, x_hi = bf16(x) and x_lo = bf16(x - x_hi), and a
// product a.b is evaluated as three bf16 MFMAs, a_hi.b_hi + a_hi.b_lo +
// a_lo.b_hi, accumulated in fp32: what is dropped (a_lo.b_lo and the rounding
// of the low terms) is about 2^-16 of |a.b|.  Same structure as the bf16
// kernels; every staged tile and every register operand exists as a hi and a
// lo copy, and outputs are stored as fp32.
// ===========================================================================
template <int R>
struct BlkF {            // R rows x 8 fp32 features (raw bits)
    u32x4 a[R], b[R];    // features 0..3 and 4..7 of row i
};

template <int R>
__device__ __forceinline__ void load_blk_f32(BlkF<R>& bl, __amdgpu_buffer_rsrc_t rs, int rg,
                                             int cg, int H, int h, int D) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const uint32_t off = uint32_t((((rg * R + i) * H + h) * D + cg * 8) * 4);
        bl.a[i] = buf_load16(rs, off);
        bl.b[i] = buf_load16(rs, off + 16);
    }
}

// 8 fp32 values (two 16-byte pieces) -> their bf16 hi and lo terms
__device__ __forceinline__ void split8(u32x4 a, u32x4 b, u32x4& hi, u32x4& lo) {
    const float f[8] = {__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]),
                        __uint_as_float(a[3]), __uint_as_float(b[0]), __uint_as_float(b[1]),
                        __uint_as_float(b[2]), __uint_as_float(b[3])};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t hh = cvt_bf2(f[2 * m], f[2 * m + 1]);
        hi[m] = hh;
        lo[m] = cvt_bf2(f[2 * m] - bf_lo(hh), f[2 * m + 1] - bf_hi(hh));
    }
}

template <int D, int DVW, int R, int NT, int NPER>
__device__ __forceinline__ void load_kv_f32(BlkF<R> (&pre)[NPER], __amdgpu_buffer_rsrc_t rk,
                                            __amdgpu_buffer_rsrc_t rv, int vcg0, int H, int h) {
    using KS = KVStage<D, DVW, R, NT>;
    const int wbase = wave_id() * 64;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int b0 = wbase + i * NT;                      // wave-uniform
        if constexpr (NPER * NT > KS::NBK + KS::NBV)
            if (b0 >= KS::NBK + KS::NBV) break;
        const bool is_v = b0 >= KS::NBK;
        const int wk = b0 + lane, wv = b0 - KS::NBK + lane;
        const int rg = is_v ? wv / KS::NCGV : wk / KS::NCGK;
        const int cg = is_v ? vcg0 + wv % KS::NCGV : wk % KS::NCGK;
        load_blk_f32<R>(pre[i], is_v ? rv : rk, rg, cg, H, h, D);
    }
}

// Registers -> LDS, each block as its hi and lo terms: K row-major
// (K_ROWS), K transposed, V transposed.
template <int D, int DVW, int R, int NT, int NPER, bool K_ROWS>
__device__ __forceinline__ void stage_kv_split(const BlkF<R> (&pre)[NPER], uint16_t* sKh,
                                               uint16_t* sKl, uint16_t* sKth, uint16_t* sKtl,
                                               uint16_t* sVth, uint16_t* sVtl) {
    using KS = KVStage<D, DVW, R, NT>;
    using ST = Stage<D, R>;
    const int wbase = wave_id() * 64;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int b0 = wbase + i * NT;                      // wave-uniform
        if constexpr (NPER * NT > KS::NBK + KS::NBV)
            if (b0 >= KS::NBK + KS::NBV) break;
        BlkR<R> hi, lo;
#pragma unroll
        for (int r = 0; r < R; ++r) split8(pre[i].a[r], pre[i].b[r], hi.r[r], lo.r[r]);
        if (b0 >= KS::NBK) {
            const int wv = b0 - KS::NBK + lane;
            store_cols<R>(sVth, hi, wv / KS::NCGV, wv % KS::NCGV, ST::LDT);
            store_cols<R>(sVtl, lo, wv / KS::NCGV, wv % KS::NCGV, ST::LDT);
        } else {
            const int wk = b0 + lane;
            if constexpr (K_ROWS) {
                store_rows<R>(sKh, hi, wk / KS::NCGK, wk % KS::NCGK, ST::LDR);
                store_rows<R>(sKl, lo, wk / KS::NCGK, wk % KS::NCGK, ST::LDR);
            }
            store_cols<R>(sKth, hi, wk / KS::NCGK, wk % KS::NCGK, ST::LDT);
            store_cols<R>(sKtl, lo, wk / KS::NCGK, wk % KS::NCGK, ST::LDT);
        }
    }
}

// a.b ~ a_hi.b_hi + a_hi.b_lo + a_lo.b_hi
__device__ __forceinline__ f32x4 mfma3(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 c) {
    c = mfma_bf16(ah, bh, c);
    c = mfma_bf16(ah, bl, c);
    return mfma_bf16(al, bh, c);
}

// Launch 1, split precision: as delta_kernel_bf16 with NP = 1.
template <int D>
__global__ __launch_bounds__(kThreads) void delta_kernel_split(
    const float* __restrict__ k, const float* __restrict__ v,
    const DeltaDesc* __restrict__ deltas, float* __restrict__ ws, int H, PlanCheck pc) {
    if (!pc.ok()) return;
    using D1 = Delta1<D, 1>;
    constexpr int R = D1::R, NKB = D1::NKB, VBW = D1::VBW, KBW = D1::KBW, DD = D * D;
    using ST = Stage<D, R>;
    constexpr int NPER = KVStage<D, D, R, kThreads>::NPER;
    __shared__ __attribute__((aligned(16))) uint16_t sKth[D * ST::LDT];
    __shared__ __attribute__((aligned(16))) uint16_t sKtl[D * ST::LDT];
    __shared__ __attribute__((aligned(16))) uint16_t sVth[D * ST::LDT];
    __shared__ __attribute__((aligned(16))) uint16_t sVtl[D * ST::LDT];

    const int h = blockIdx.x % H;
    const DeltaDesc dd = deltas[blockIdx.x / H];
    const int w = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
    const int vbw = D1::vb0(w), kbw = D1::kb0(w);

    f32x4 S[VBW][KBW];
#pragma unroll
    for (int x = 0; x < VBW; ++x)
#pragma unroll
        for (int i = 0; i < KBW; ++i) S[x][i] = zero4();

    const int nch = (dd.ntok + kChunk - 1) / kChunk;
    const int64_t row_elems = int64_t(H) * D;
    BlkF<R> pre[NPER];
    auto load = [&](int c) {
        const int64_t first = (int64_t(dd.tok0) + c * kChunk) * row_elems;
        const int rows = min(kChunk, dd.ntok - c * kChunk);   // <= 0: empty window
        load_kv_f32<D, D, R, kThreads, NPER>(pre, chunk_rsrc(k, first, 4, rows, H, D),
                                             chunk_rsrc(v, first, 4, rows, H, D), 0, H, h);
    };
    load(0);
    for (int c = 0; c < nch; ++c) {
        stage_kv_split<D, D, R, kThreads, NPER, false>(pre, nullptr, nullptr, sKth, sKtl, sVth,
                                                       sVtl);
        __syncthreads();
        load(c + 1);   // empty window past the last chunk
#pragma unroll
        for (int ks = 0; ks < kChunk / 32; ++ks) {
#pragma unroll
            for (int x = 0; x < VBW; ++x) {
                const int vb = vbw + x;
                const int vo = (vb * 16 + c16) * ST::LDT + tpos(vb * 16, ks * 32 + 4 * g);
                const u32x4 bvh = lds_u32x4(sVth + vo), bvl = lds_u32x4(sVtl + vo);
#pragma unroll
                for (int i = 0; i < KBW; ++i) {
                    const int kb = kbw + i;
                    const int ko = (kb * 16 + c16) * ST::LDT + tpos(kb * 16, ks * 32 + 4 * g);
                    S[x][i] = mfma3(lds_u32x4(sKth + ko), lds_u32x4(sKtl + ko), bvh, bvl, S[x][i]);
                }
            }
        }
        __syncthreads();
    }
    f32x4* dst = reinterpret_cast<f32x4*>(ws + ((int64_t)dd.slot * H + h) * DD);
#pragma unroll
    for (int x = 0; x < VBW; ++x)
#pragma unroll
        for (int i = 0; i < KBW; ++i) dst[((vbw + x) * NKB + kbw + i) * 64 + lane] = S[x][i];
}

// The outputs of one wave for one chunk, split precision (see out_tiles).
template <int D, int TB, int VBH>
__device__ __forceinline__ void out_tiles_split(const uint16_t* sKh, const uint16_t* sKl,
                                                const uint16_t* sVth, const uint16_t* sVtl,
                                                const uint16_t* sSh, const uint16_t* sSl,
                                                const u32x4 (&qh)[D / 32],
                                                const u32x4 (&ql)[D / 32], int vb0, int g,
                                                int c16, f32x4 (&acc)[VBH]) {
    constexpr int NKS = D / 32;
    constexpr int LDR = Stage<D, 4>::LDR, LDT = Stage<D, 4>::LDT;
    f32x4 p[TB + 1];
#pragma unroll
    for (int ub = 0; ub <= TB; ++ub) p[ub] = zero4();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int ub = 0; ub <= TB; ++ub) {
            const int o = (ub * 16 + c16) * LDR + ks * 32 + 8 * g;
            p[ub] = mfma3(lds_u32x4(sKh + o), lds_u32x4(sKl + o), qh[ks], ql[ks], p[ub]);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)   // causal mask inside the diagonal tile: u <= t
        if (4 * g + j > c16) p[TB][j] = 0.f;
    u32x2 ph[4], pl[4];
#pragma unroll
    for (int ub = 0; ub < 4; ++ub) {
        if (ub <= TB) {
            const uint32_t h01 = cvt_bf2(p[ub][0], p[ub][1]), h23 = cvt_bf2(p[ub][2], p[ub][3]);
            ph[ub] = u32x2{h01, h23};
            pl[ub] = u32x2{cvt_bf2(p[ub][0] - bf_lo(h01), p[ub][1] - bf_hi(h01)),
                           cvt_bf2(p[ub][2] - bf_lo(h23), p[ub][3] - bf_hi(h23))};
        } else {
            ph[ub] = pl[ub] = u32x2{0u, 0u};
        }
    }
#pragma unroll
    for (int x = 0; x < VBH; ++x) acc[x] = zero4();
    // inter-chunk: O^T += S^T Q^T
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int x = 0; x < VBH; ++x) {
            const int f = (vb0 + x) * 16 + c16;
            const int o = f * LDR + scol<D>(f, ks * 32 + 8 * g);
            acc[x] = mfma3(lds_u32x4(sSh + o), lds_u32x4(sSl + o), qh[ks], ql[ks], acc[x]);
        }
    // intra-chunk: O^T += V^T P^T
#pragma unroll
    for (int pp = 0; pp <= TB / 2; ++pp) {
        const u32x4 bh = cat2(ph[2 * pp], ph[2 * pp + 1]), bl = cat2(pl[2 * pp], pl[2 * pp + 1]);
#pragma unroll
        for (int x = 0; x < VBH; ++x) {
            const int vb = vb0 + x;
            const int o = (vb * 16 + c16) * LDT + tpos(vb * 16, pp * 32 + 4 * g);
            acc[x] = mfma3(lds_u32x4(sVth + o), lds_u32x4(sVtl + o), bh, bl, acc[x]);
        }
    }
}

// Launch 3, split precision: as output_kernel_bf16 (same launch shape O3).
template <int D, class O3, bool FUSED>
__global__ __launch_bounds__(O3::NT) void output_kernel_split(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const BlockDesc* __restrict__ blocks, const ScanDesc* __restrict__ scans,
    const float* __restrict__ ws, float* __restrict__ final_state,
    const float* __restrict__ ext_state, float* __restrict__ out, int H, int n_items,
    PlanCheck pc) {
    if (!pc.ok()) return;
    constexpr int R = O3::R, NT = O3::NT, NP = O3::NP_, DV = O3::DV;
    using ST = Stage<D, R>;
    constexpr int NKB = O3::NKB, NVB = O3::NVB, NKS = O3::NKS, VBH = O3::VBH, TPW = O3::TPW;
    constexpr int NPER = KVStage<D, DV, R, NT>::NPER;
    constexpr int LDR = ST::LDR, LDT = ST::LDT;
    __shared__ __attribute__((aligned(16))) uint16_t sKh[kChunk * LDR];
    __shared__ __attribute__((aligned(16))) uint16_t sKl[kChunk * LDR];
    __shared__ __attribute__((aligned(16))) uint16_t sKth[D * LDT];
    __shared__ __attribute__((aligned(16))) uint16_t sKtl[D * LDT];
    __shared__ __attribute__((aligned(16))) uint16_t sVth[DV * LDT];
    __shared__ __attribute__((aligned(16))) uint16_t sVtl[DV * LDT];
    __shared__ __attribute__((aligned(16))) uint16_t sSh[DV * LDR];
    __shared__ __attribute__((aligned(16))) uint16_t sSl[DV * LDR];

    int item, part;
    split_id<NP>(blockIdx.x, item, part);
    if (item >= n_items) return;   // whole workgroup: padding of the split grid
    const int h = item % H;
    const BlockDesc bd = blocks[item / H];
    const int w = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
    const int tb = w & 3, hv = w >> 2;
    const int vbo = O3::vb_own(w), kbo = O3::kb0(w);
    const int vbg = part * NVB + vbo;

    const int nch = (bd.ntok + kChunk - 1) / kChunk;
    const int64_t row_elems = int64_t(H) * D;
    const int trow = tb * 16 + c16;
    const uint32_t qoff = uint32_t(((trow * H + h) * D + 8 * g) * 4);
    const uint32_t ooff =
        uint32_t(((trow * H + h) * D + part * DV + hv * VBH * 16 + 4 * g) * 4);
    const int vcg0 = part * (DV / 8);

    BlkF<R> kv[NPER];
    u32x4 qa[NKS], qb[NKS], qh[NKS], ql[NKS];
    auto load = [&](int c) {
        const int64_t first = (int64_t(bd.tok0) + c * kChunk) * row_elems;
        const int rows = min(kChunk, bd.ntok - c * kChunk);   // <= 0: empty window
        load_kv_f32<D, DV, R, NT, NPER>(kv, chunk_rsrc(k, first, 4, rows, H, D),
                                        chunk_rsrc(v, first, 4, rows, H, D), vcg0, H, h);
        const auto rq = chunk_rsrc(q, first, 4, rows, H, D);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            qa[ks] = buf_load16(rq, qoff + ks * 128);
            qb[ks] = buf_load16(rq, qoff + ks * 128 + 16);
        }
    };
    // first chunk's loads before the initial state's (see output_kernel_bf16)
    load(0);

    f32x4 S[TPW];
    {
        int tix[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) tix[i] = vbg * NKB + kbo + i;
        block_init_state<D, TPW, FUSED>(S, tix, bd, scans, ws, final_state, ext_state, H, h,
                                        lane);
    }

    auto publish_and_stage = [&]() {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const f32x4 s = S[i];
            const uint32_t h01 = cvt_bf2(s[0], s[1]), h23 = cvt_bf2(s[2], s[3]);
            const uint32_t l01 = cvt_bf2(s[0] - bf_lo(h01), s[1] - bf_hi(h01));
            const uint32_t l23 = cvt_bf2(s[2] - bf_lo(h23), s[3] - bf_hi(h23));
            const int off = (vbo * 16 + c16) * LDR + scol<D>(vbo * 16 + c16, (kbo + i) * 16 + 4 * g);
            *reinterpret_cast<u32x2*>(sSh + off) = u32x2{h01, h23};
            *reinterpret_cast<u32x2*>(sSl + off) = u32x2{l01, l23};
        }
        stage_kv_split<D, DV, R, NT, NPER, true>(kv, sKh, sKl, sKth, sKtl, sVth, sVtl);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) split8(qa[ks], qb[ks], qh[ks], ql[ks]);
    };
    // rotated loop, as in output_kernel_bf16: chunk c + 1 is staged after
    // chunk c's output stores, and the entry leaves no loads outstanding
    publish_and_stage();
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    for (int c = 0; c < nch; ++c) {
        __syncthreads();
        load(c + 1);

        const int rows = min(kChunk, bd.ntok - c * kChunk);
        const int64_t first = (int64_t(bd.tok0) + c * kChunk) * row_elems;
        f32x4 acc[VBH];
        switch (tb) {
            case 0: out_tiles_split<D, 0, VBH>(sKh, sKl, sVth, sVtl, sSh, sSl, qh, ql, hv * VBH, g, c16, acc); break;
            case 1: out_tiles_split<D, 1, VBH>(sKh, sKl, sVth, sVtl, sSh, sSl, qh, ql, hv * VBH, g, c16, acc); break;
            case 2: out_tiles_split<D, 2, VBH>(sKh, sKl, sVth, sVtl, sSh, sSl, qh, ql, hv * VBH, g, c16, acc); break;
            default: out_tiles_split<D, 3, VBH>(sKh, sKl, sVth, sVtl, sSh, sSl, qh, ql, hv * VBH, g, c16, acc); break;
        }
        {
            const auto ro = chunk_rsrc(out, first, 4, rows, H, D);
#pragma unroll
            for (int x = 0; x < VBH; ++x) buf_store16(ro, ooff + x * 64, acc[x]);
        }
        if (c + 1 >= nch) break;
#pragma unroll
        for (int ks = 0; ks < kChunk / 32; ++ks) {
            const int vo = (vbo * 16 + c16) * LDT + tpos(vbo * 16, ks * 32 + 4 * g);
            const u32x4 bvh = lds_u32x4(sVth + vo), bvl = lds_u32x4(sVtl + vo);
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int ko = ((kbo + i) * 16 + c16) * LDT + tpos((kbo + i) * 16, ks * 32 + 4 * g);
                S[i] = mfma3(lds_u32x4(sKth + ko), lds_u32x4(sKtl + ko), bvh, bvl, S[i]);
            }
        }
        __syncthreads();
        publish_and_stage();
    }
}

// ===========================================================================
// View-state and view K/V export: plain vectorised copy of 16-byte pieces.
// ===========================================================================
__global__ __launch_bounds__(kThreads) void copy_kernel(const f32x4* __restrict__ src,
                                                        f32x4* __restrict__ dst, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n4) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
bool supported_dims(int32_t d_k, int32_t d_v) {
    return d_k == d_v && (d_k == 64 || d_k == 128);
}

// The two-launch form trades the prefix launch (about 3 us of launch and
// memory latency, whatever the pass) for workspace reads at the start of
// output workgroups, bound by one CU's load rate (a block late in a long view
// sums a dozen 16 KB slots before its first chunk).  Measured on MI355X,
// pass us with three / two launches: 628 tokens (fp32) 16.9 / 15.7; 7,400
// tokens 29.1-29.4 / 28.2 (58 MB of slot reads); four requests of 27,187
// tokens 79.3 / 77.0 (113 MB); one view of 18,000 with 256 branches
// 100.9 / 131.1 (1.25 GB).
constexpr double kTwoLaunchReadBytes = 128.0 * 1024 * 1024;
// Polls of a single-launch wait before it gives up (each poll is a device-
// coherent load plus a short sleep: a few tenths of a second in all, four
// orders of magnitude above a wait in a normal pass).
constexpr int32_t kSpinLimit = 1 << 18;
bool two_launch_pays(const la_pass_info& info, int32_t H, int32_t d) {
    return double(info.fused_slot_reads) * H * d * d * 4 <= kTwoLaunchReadBytes;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Every launch's grid, in work-items, must fit the 32-bit dispatch size.
template <int D>
bool grids_fit(const la_pass_info& info, int32_t H) {
    constexpr int64_t kMax = (int64_t(1) << 32) - 1;
    using O3 = typename LaunchCfg<D>::O3;
    using O3S = typename LaunchCfg<D>::O3S;
    const int64_t l1 = split_grid<LaunchCfg<D>::DELTA_NP>(int64_t(info.n_delta) * H) * kThreads;
    const int64_t l2 = int64_t(info.n_scan) * H * (D * D);
    const int64_t l3 = split_grid<O3::NP_>(int64_t(info.n_blocks) * H) *
                       (O3::NT > kThreads ? O3::NT : kThreads);
    const int64_t l3s = split_grid<O3S::NP_>(int64_t(info.n_blocks) * H) *
                        (O3S::NT > kThreads ? O3S::NT : kThreads);
    return l1 <= kMax && l2 <= kMax && l3 <= kMax && l3s <= kMax;
}

template <int D>
la_status launch_all(int32_t stages, bool fused, const void* q, const void* k, const void* v,
                     la_dtype dtype, int32_t H, const la_pass_info& info, const int32_t* plan,
                     const float* ext_state, void* out, float* final_state, float* ws,
                     hipStream_t st, PlanCheck pc) {
    const int32_t off_blocks = LA_PLAN_HEADER_WORDS;
    const int32_t off_delta = off_blocks + info.n_blocks * LA_PLAN_BLOCK_WORDS;
    const int32_t off_scan = off_delta + info.n_delta * LA_PLAN_DELTA_WORDS;
    const auto* blocks = reinterpret_cast<const BlockDesc*>(plan + off_blocks);
    const auto* deltas = reinterpret_cast<const DeltaDesc*>(plan + off_delta);
    const auto* scans = reinterpret_cast<const ScanDesc*>(plan + off_scan);
    const dim3 blk(kThreads);
    if ((stages & LA_STAGE_STATES) && info.n_delta > 0) {
        const int items = info.n_delta * H;
        constexpr int NP = LaunchCfg<D>::DELTA_NP;
        if (dtype == LA_BF16)
            hipLaunchKernelGGL((delta_kernel_bf16<D, NP>), dim3(unsigned(split_grid<NP>(items))),
                               blk, 0, st, static_cast<const uint16_t*>(k),
                               static_cast<const uint16_t*>(v), deltas, ws, H, items, pc);
        else if (dtype == LA_F32_SPLIT)
            hipLaunchKernelGGL(delta_kernel_split<D>, dim3(unsigned(items)), blk, 0, st,
                               static_cast<const float*>(k), static_cast<const float*>(v),
                               deltas, ws, H, pc);
        else
            hipLaunchKernelGGL(delta_kernel_f32<D>, dim3(unsigned(items)), blk, 0, st,
                               static_cast<const float*>(k), static_cast<const float*>(v), deltas,
                               ws, H, pc);
        if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    }
    if ((stages & LA_STAGE_PREFIX) && !fused && info.n_scan > 0) {
        const int64_t wgs = int64_t(info.n_scan) * H * (D * D / kThreads);
        if (wgs >= kPrefixWideGroups)
            hipLaunchKernelGGL((prefix_kernel<D, 4, 8>), dim3(unsigned(wgs / 4)), blk, 0, st,
                               scans, ws, final_state, H, pc);
        else
            hipLaunchKernelGGL((prefix_kernel<D, 1, 32>), dim3(unsigned(wgs)), blk, 0, st,
                               scans, ws, final_state, H, pc);
        if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    }
    if ((stages & LA_STAGE_OUTPUT) && info.n_blocks > 0) {
        const int items = info.n_blocks * H;
        using O3 = typename LaunchCfg<D>::O3;
        const dim3 g3(unsigned(split_grid<O3::NP_>(items)));
        if (dtype == LA_BF16) {
            auto kern = fused ? output_kernel_bf16<D, O3, true> : output_kernel_bf16<D, O3, false>;
            hipLaunchKernelGGL(kern, g3, dim3(O3::NT), 0, st, static_cast<const uint16_t*>(q),
                               static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                               blocks, scans, ws, final_state, ext_state,
                               static_cast<uint16_t*>(out), H, items, pc);
        } else if (dtype == LA_F32_SPLIT) {
            using O3S = typename LaunchCfg<D>::O3S;
            auto kern = fused ? output_kernel_split<D, O3S, true> : output_kernel_split<D, O3S, false>;
            const dim3 g3s(unsigned(split_grid<O3S::NP_>(items)));
            hipLaunchKernelGGL(kern, g3s, dim3(O3S::NT), 0, st, static_cast<const float*>(q),
                               static_cast<const float*>(k), static_cast<const float*>(v), blocks,
                               scans, ws, final_state, ext_state, static_cast<float*>(out), H,
                               items, pc);
        } else {
            auto kern = fused ? output_kernel_f32<D, true> : output_kernel_f32<D, false>;
            hipLaunchKernelGGL(kern, dim3(unsigned(items)), blk, 0, st,
                               static_cast<const float*>(q), static_cast<const float*>(k),
                               static_cast<const float*>(v), blocks, scans, ws, final_state,
                               ext_state, static_cast<float*>(out), H, pc);
        }
        if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    }
    return LA_OK;
}

// ---------------------------------------------------------------------------
// Built-in scratch memory for la_scan_packed_noalloc (callers that cannot
// allocate).  One copy per GPU; host code never uses the array's name as an
// address: each device's copy is found once with hipGetSymbolAddress and that
// pointer is what the kernels receive, exactly like a caller's workspace.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
// the first bytes of the array are cleared once per GPU at set-up
constexpr size_t kScratchClearBytes = size_t(1) << 20;

struct ScratchDevice {
    std::once_flag once;
    void* ptr = nullptr;
    la_status status = LA_ERR_HIP;
};
ScratchDevice g_scratch[kMaxScratchDevices];

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(f32x4* __restrict__ p, int64_t n4) {
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i < n4) p[i] = zero4();
}

// The current device's copy of `scratch`; set-up (address, clearing) on the
// first call for that device, with the device current.
la_status scratch_for_current_device(hipStream_t st, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return LA_ERR_HIP;
    ScratchDevice& sd = g_scratch[dev];
    std::call_once(sd.once, [&]() {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return;
        const int64_t n4 = int64_t(kScratchClearBytes / 16);
        hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned((n4 + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, st, static_cast<f32x4*>(p), n4);
        if (hipGetLastError() != hipSuccess) return;
        sd.ptr = p;
        sd.status = LA_OK;
    });
    if (sd.status != LA_OK) return sd.status;
    *out = sd.ptr;
    return LA_OK;
}

// Bytes of the workspace before the old path's block states: the header
// (status word) every form shares.
constexpr size_t kWsHeader = piece::kHeaderBytes;

bool info_matches(const la_pass_info& info) {
    return uint32_t(info.info_check) == la_info_checksum(&info);
}

}  // namespace

namespace piece {
// The prefix launch over the piece path's slots (views' totals go to
// final_state); every slot, the first included, becomes the sum from zero of
// the slots up to it.
la_status launch_prefix(const int32_t* scans, int32_t n_scan, float* slots, float* final_state,
                        int32_t H, hipStream_t st, const int32_t* plan, int* hdr, int hash) {
    const PlanCheck pc{plan, hdr, hash};
    const auto* sc = reinterpret_cast<const ScanDesc*>(scans);
    const int64_t wgs = int64_t(n_scan) * H * (64 * 64 / kThreads);
    if (wgs >= kPrefixWideGroups)
        hipLaunchKernelGGL((prefix_kernel<64, 4, 8, true>), dim3(unsigned(wgs / 4)),
                           dim3(kThreads), 0, st, sc, slots, final_state, H, pc);
    else
        hipLaunchKernelGGL((prefix_kernel<64, 1, 32, true>), dim3(unsigned(wgs)), dim3(kThreads),
                           0, st, sc, slots, final_state, H, pc);
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}
}  // namespace piece

namespace {
}  // namespace

extern "C" la_status la_scan_workspace_size(const la_pass_info* info, int32_t H, int32_t d_k,
                                            int32_t d_v, la_dtype dtype, size_t* bytes) {
    if (!info || !bytes || H < 1 || info->n_delta < 0 || info->piece_slots < 0)
        return LA_ERR_INVALID_ARG;
    if (!supported_dims(d_k, d_v) || (dtype != LA_F32 && dtype != LA_BF16 && dtype != LA_F32_SPLIT))
        return LA_ERR_UNSUPPORTED;
    if (piece::applies(d_k, dtype))
        *bytes = piece::workspace_bytes(*info, H);
    else
        *bytes = kWsHeader +
                 size_t(info->n_delta) * size_t(H) * size_t(d_k) * size_t(d_v) * sizeof(float);
    return LA_OK;
}

extern "C" la_status la_scan_packed_stages(int32_t stages, const void* q, const void* k,
                                           const void* v, la_dtype dtype, int32_t H,
                                           int32_t d_k, int32_t d_v, const la_pass_info* info,
                                           const int32_t* plan, const float* ext_state,
                                           int32_t n_ext, void* out, float* final_state,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream) {
    constexpr int32_t kForms = LA_FORM_ONE_LAUNCH | LA_FORM_TWO_LAUNCH | LA_FORM_THREE_LAUNCH;
    if (!info || (stages & ~(LA_STAGE_ALL | kForms | LA_DEBUG_FORCE_TIMEOUT | LA_DEBUG_ORDERED)) ||
        !(stages & LA_STAGE_ALL) || __builtin_popcount(unsigned(stages & kForms)) > 1)
        return LA_ERR_INVALID_ARG;
    // an la_pass_info whose fields were edited, or mixed from two passes
    if (!info_matches(*info)) return LA_ERR_INVALID_ARG;
    if (dtype != LA_F32 && dtype != LA_BF16 && dtype != LA_F32_SPLIT) return LA_ERR_UNSUPPORTED;
    if (!supported_dims(d_k, d_v) || info->chunk != LA_CHUNK) return LA_ERR_UNSUPPORTED;
    if (H < 1 || info->n_tokens < 0 || info->n_blocks < 0 || info->n_delta < 0 ||
        info->n_scan < 0 || info->n_views < 0 || info->n_ext < 0 || n_ext < 0)
        return LA_ERR_INVALID_ARG;
    if (info->n_tokens == 0) return LA_OK;
    if (int64_t(info->n_tokens) * H * d_k >= (int64_t(1) << 40)) return LA_ERR_INVALID_ARG;
    // a chunk window (64 token rows of all heads) must fit a 32-bit buffer range
    if (int64_t(kChunk) * H * d_k * 4 >= (int64_t(1) << 31)) return LA_ERR_INVALID_ARG;
    if (!(d_k == 64 ? grids_fit<64>(*info, H) : grids_fit<128>(*info, H)))
        return LA_ERR_INVALID_ARG;
    if (!q || !k || !v || !out || !plan) return LA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return LA_ERR_INVALID_ARG;
    if (info->n_views > 0 && !final_state) return LA_ERR_INVALID_ARG;
    if (info->n_ext > 0 && (!ext_state || n_ext < info->n_ext)) return LA_ERR_INVALID_ARG;
    // the states and the workspace are read and written as fp32 (16-byte rows
    // for the workspace), the plan as int32
    if ((final_state && !aligned4(final_state)) || (ext_state && !aligned4(ext_state)) ||
        (workspace && !aligned16(workspace)) || !aligned4(plan))
        return LA_ERR_INVALID_ARG;
    // final_state is written while ext_state is read (by the same launch in the
    // two-launch form): the two must not overlap
    if (final_state && ext_state && info->n_views > 0 && n_ext > 0) {
        const uintptr_t st = uintptr_t(H) * d_k * d_v * sizeof(float);
        const uintptr_t f0 = reinterpret_cast<uintptr_t>(final_state);
        const uintptr_t e0 = reinterpret_cast<uintptr_t>(ext_state);
        if (f0 < e0 + uintptr_t(n_ext) * st && e0 < f0 + uintptr_t(info->n_views) * st)
            return LA_ERR_INVALID_ARG;
    }
    size_t need = 0;
    la_status stw = la_scan_workspace_size(info, H, d_k, d_v, dtype, &need);
    if (stw != LA_OK) return stw;
    if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (piece::applies(d_k, dtype)) {
        const int form = (stages & LA_FORM_TWO_LAUNCH)     ? 2
                         : (stages & LA_FORM_THREE_LAUNCH) ? 3
                                                           : 1;
        const bool force = (stages & LA_DEBUG_FORCE_TIMEOUT) != 0;
        return piece::launch(stages & LA_STAGE_ALL, form, q, k, v, H, *info, plan, ext_state,
                             out, final_state, workspace, st, force ? 16 : kSpinLimit, force,
                             (stages & LA_DEBUG_ORDERED) != 0);
    }
    if (stages & (LA_FORM_ONE_LAUNCH | LA_DEBUG_FORCE_TIMEOUT | LA_DEBUG_ORDERED))
        return LA_ERR_UNSUPPORTED;
    int* hdr = static_cast<int*>(workspace);
    float* ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + kWsHeader);
    const PlanCheck pc{plan, hdr, info->plan_hash};
    const bool fused = (stages & LA_FORM_TWO_LAUNCH) ||
                       (!(stages & LA_FORM_THREE_LAUNCH) && two_launch_pays(*info, H, d_k));
    if (d_k == 64)
        return launch_all<64>(stages, fused, q, k, v, dtype, H, *info, plan, ext_state, out,
                              final_state, ws, st, pc);
    return launch_all<128>(stages, fused, q, k, v, dtype, H, *info, plan, ext_state, out,
                           final_state, ws, st, pc);
}

extern "C" la_status la_scan_launches(const la_pass_info* info, int32_t H, int32_t d_k,
                                      int32_t d_v, la_dtype dtype, int32_t* n_launches) {
    if (!info || !n_launches || H < 1) return LA_ERR_INVALID_ARG;
    if (!supported_dims(d_k, d_v)) return LA_ERR_UNSUPPORTED;
    if (piece::applies(d_k, dtype))
        *n_launches = 1;
    else
        *n_launches = two_launch_pays(*info, H, d_k) ? 2 : 3;
    return LA_OK;
}

extern "C" la_status la_scan_status(const void* workspace, size_t workspace_bytes,
                                    int32_t* status, int32_t clear, void* stream) {
    if (!workspace || !status || workspace_bytes < kWsHeader) return LA_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t v = 0;
    const int32_t* src = static_cast<const int32_t*>(workspace) + piece::kStatusWord;
    if (hipMemcpyAsync(&v, src, sizeof(v), hipMemcpyDeviceToHost, st) != hipSuccess)
        return LA_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return LA_ERR_HIP;
    if (clear && v != 0) {
        const int32_t zero = 0;
        if (hipMemcpyAsync(const_cast<int32_t*>(src), &zero, sizeof(zero), hipMemcpyHostToDevice,
                           st) != hipSuccess ||
            hipStreamSynchronize(st) != hipSuccess)
            return LA_ERR_HIP;
    }
    *status = v;
    return LA_OK;
}

extern "C" la_status la_scan_packed(const void* q, const void* k, const void* v, la_dtype dtype,
                                    int32_t H, int32_t d_k, int32_t d_v,
                                    const la_pass_info* info, const int32_t* plan,
                                    const float* ext_state, int32_t n_ext, void* out,
                                    float* final_state, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return la_scan_packed_stages(LA_STAGE_ALL, q, k, v, dtype, H, d_k, d_v, info, plan, ext_state,
                                 n_ext, out, final_state, workspace, workspace_bytes, stream);
}

extern "C" la_status la_export_view_state(const float* final_state, int32_t view_row,
                                          int32_t n_views, int32_t H, int32_t d_k, int32_t d_v,
                                          float* dst, void* stream) {
    if (!final_state || !dst || H < 1 || n_views < 1 || view_row < 0 || view_row >= n_views)
        return LA_ERR_INVALID_ARG;
    if (!supported_dims(d_k, d_v)) return LA_ERR_UNSUPPORTED;
    if (!aligned16(final_state) || !aligned16(dst)) return LA_ERR_INVALID_ARG;
    const int64_t n = int64_t(H) * d_k * d_v;
    const float* src = final_state + int64_t(view_row) * n;
    if (dst < src + n && src < dst + n) return LA_ERR_INVALID_ARG;
    const int64_t n4 = n / 4;
    const unsigned grid = unsigned((n4 + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<const f32x4*>(src),
                       reinterpret_cast<f32x4*>(dst), n4);
    if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    return LA_OK;
}

extern "C" la_status la_export_view_kv(const void* k, const void* v, la_dtype dtype,
                                       int32_t n_tokens, int32_t H, int32_t d, int32_t tok0,
                                       int32_t n_tok, void* dst_k, void* dst_v, void* stream) {
    if (!k || !v || !dst_k || !dst_v || H < 1 || n_tokens < 1 || tok0 < 0 || n_tok < 1 ||
        int64_t(tok0) + n_tok > n_tokens)
        return LA_ERR_INVALID_ARG;
    if (dtype != LA_BF16 && dtype != LA_F32) return LA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    if (!aligned16(k) || !aligned16(v) || !aligned16(dst_k) || !aligned16(dst_v))
        return LA_ERR_INVALID_ARG;
    const int64_t row = int64_t(H) * d * (dtype == LA_BF16 ? 2 : 4);   // bytes per token
    const int64_t bytes = row * n_tok;
    const char* sk = static_cast<const char*>(k) + row * tok0;
    const char* sv = static_cast<const char*>(v) + row * tok0;
    char* dk = static_cast<char*>(dst_k);
    char* dv = static_cast<char*>(dst_v);
    auto overlap = [bytes](const char* a, const char* b) { return a < b + bytes && b < a + bytes; };
    if (overlap(sk, dk) || overlap(sk, dv) || overlap(sv, dk) || overlap(sv, dv) ||
        overlap(dk, dv))
        return LA_ERR_INVALID_ARG;
    const int64_t n4 = bytes / 16;
    if ((n4 + kThreads - 1) / kThreads > int64_t(UINT32_MAX)) return LA_ERR_INVALID_ARG;
    const unsigned grid = unsigned((n4 + kThreads - 1) / kThreads);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(kThreads), 0, st,
                       reinterpret_cast<const f32x4*>(sk), reinterpret_cast<f32x4*>(dk), n4);
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(kThreads), 0, st,
                       reinterpret_cast<const f32x4*>(sv), reinterpret_cast<f32x4*>(dv), n4);
    if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    return LA_OK;
}

extern "C" la_status la_scan_packed_noalloc(const void* q, const void* k, const void* v,
                                            la_dtype dtype, int32_t H, int32_t d_k,
                                            int32_t d_v, const la_pass_info* info,
                                            const int32_t* plan, const float* ext_state,
                                            int32_t n_ext, void* out, float* final_state,
                                            void* stream) {
    if (!info) return LA_ERR_INVALID_ARG;
    size_t need = 0;
    const la_status sz = la_scan_workspace_size(info, H, d_k, d_v, dtype, &need);
    if (sz != LA_OK) return sz;
    if (need > size_t(LA_NOALLOC_SCRATCH_BYTES)) return LA_ERR_TOO_LARGE;
    void* ws = nullptr;
    const la_status ss = scratch_for_current_device(static_cast<hipStream_t>(stream), &ws);
    if (ss != LA_OK) return ss;
    return la_scan_packed_stages(LA_STAGE_ALL, q, k, v, dtype, H, d_k, d_v, info, plan,
                                 ext_state, n_ext, out, final_state, ws,
                                 size_t(LA_NOALLOC_SCRATCH_BYTES), stream);
}
