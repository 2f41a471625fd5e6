// Piece path of the packed chunked causal linear-attention scan: d = 64,
// bf16 inputs, gfx950 (MI355X).
//
// Source: "Serving 0.88M TPS from Two RTXs and Mac Minis", section "Kernels"
// (linear attention in 64-token chunks with a few 64x64 matrix products
// each; one scan covers every view of a pass) and section "Long Requests"
// (branches start from their view's state).  Per head, fp32 state S (64x64):
//     S_t = S_{t-1} + k_t^T v_t,     o_t = q_t S_t.
//
// Decomposition.  A segment (a view or a branch) is cut into blocks of
// LA_PIECE_BLOCK_CHUNKS = 8 chunks, a block into up to four pieces of
// LA_PIECE_CHUNKS = 2 chunks.  One workgroup of four waves takes a block
// and a head; wave w owns piece w end to end: it loads that piece's k, v
// and q, keeps whole 64x64 states in its own registers, and computes every
// output feature of its tokens, so the chunk loop has no workgroup barrier.
// Branches whose only block is one piece are packed into workgroups of their
// own, four waves of them: two branches of at most one chunk share a wave,
// a branch of two chunks has one alone.
//
// Arithmetic, identical in every form (same device functions, same order):
//   A_w   = sum over the piece's chunks of K_c^T V_c (MFMA accumulation,
//           chunk 1 before chunk 0), the piece's own state;
//   E_w   = 0 + A_0 + ... + A_{w-1} (fp32, left to right), the block's
//           state before piece w;
//   A_b   = E_{n-1} + A_{n-1}, the block's own state (n pieces);
//   own_j = 0 + A_b(0) + ... + A_b(j-1), the segment's state before block j;
//   S_b   = seed (a branch: its view's total own; a shard branch: ext_state;
//           a view: 0), then += own_j if j > 0;
//   S     = S_b + E_w, the state piece w starts from;
//   O_0   = tril(Q_0 K_0^T) V_0 + Q_0 S,
//   O_1   = tril(Q_1 K_1^T) V_1 + (Q_1 K_0^T) V_0 + Q_1 S  (MFMA accumulation
//           in that order; scores enter the value products as bf16, S as
//           S_hi + S_lo, two bf16 terms, which keeps the state's fp32
//           precision in the product at no memory cost).
// The terms without S need only the piece's own q, k, v: a workgroup
// computes them while the blocks before it publish their states, and adds
// Q S once S_b is known.
//
// Forms (they differ only in how own_j and the seed reach a workgroup):
//   three launches  states -> prefix (the shared prefix kernel, in place)
//                   -> outputs reading own_j and the view total from slots;
//   two launches    states -> outputs summing the slots themselves;
//   one launch      each workgroup computes A_b, publishes it, and obtains
//                   own_j from its predecessors in the same launch (a
//                   decoupled look-back: the nearest predecessor that has
//                   published its inclusive prefix, then the aggregates after
//                   it, added left to right, so the bits do not depend on
//                   timing), publishes its own inclusive prefix where a
//                   later workgroup reads it (a view's total; every block
//                   when the work comes by ticket), then computes its
//                   outputs from the k and v it already holds.  A branch's
//                   seed is its view's total, read once the view's last
//                   block has published it, or, when the whole grid is
//                   resident, summed by the branch's workgroup itself from
//                   the view's block states (the same fold, so the same
//                   bits).  k and v are read from HBM once per pass.
//
// Single-launch coordination.  A workgroup only waits for work that comes
// before its own.  When the whole grid is resident on the device at once
// (the launch checks the occupancy), the workgroup index is the work;
// otherwise workgroups take tickets from a counter in the workspace header,
// so a workgroup only ever waits for tickets taken before its own (running
// workgroups): forward progress never depends on the dispatch order.
// Published states and flags are written and read with device-coherent
// accesses (sc1; a state published from the reader's own XCD is read through
// that XCD's L2), stores are drained (s_waitcnt) before the flag that
// announces them, and every wait is bounded: past the spin limit the
// workgroup records LA_ERR_TIMEOUT in the header and carries on, so every
// wave reaches the end of the kernel.  A workgroup is counted out as soon
// as it is done with the flags (before its outputs); the last one counted
// clears the flags and resets the counters for the next pass.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "linattn.h"
#include "piece.h"
#include "tiles.h"

namespace {

constexpr int PD = 64;                       // head dim of this path
constexpr int PLD = 80;                      // staged row stride (elements): 160-byte rows
constexpr int kStageElems = kChunk * PLD;    // one 64-row tile
constexpr int kTiles = 16;                   // 16x16 tiles of a 64x64 state
constexpr int kStateBytes = PD * PD * 4;     // one state, fp32
constexpr int kWaitLgkm0 = 0xC07F;           // s_waitcnt lgkmcnt(0), others at max
constexpr uint64_t kFlagA = 0x7FF44C41464C0001ull;   // aggregate published (NaN payload)
constexpr uint64_t kFlagP = 0x7FF44C41464C0002ull;   // inclusive prefix published
constexpr int kAuxCoherent = 16;             // buffer-op cache policy: sc1 (device scope)
constexpr int kAuxL2 = 1;                    // sc0: past the CU's L1, served by the XCD's L2
constexpr uint64_t kFlagXcd = 0xF00ull;      // flag bits naming the publisher's XCD
constexpr int kHwRegXccId = (3 << 11) | 20;  // s_getreg operand: XCC_ID bits 3:0

enum Mode { kStates = 0, kOut3 = 1, kOut2 = 2, kFused = 3 };

struct PBlock {
    int tok0, ntok, slot, seed, seg, slot0, j, final_row;
};
struct PItem {
    int kind, n, b[8], pad0, pad1;
};
struct PItemBlock {                // a block item: its block copied in
    int kind, n, b0, unused;
    PBlock blk;
};
static_assert(sizeof(PItem) == sizeof(PItemBlock), "one item size");
struct PScan {
    int first_slot, n_slots, final_row, seg;
};

struct PArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* plan;
    const PBlock* blocks;
    const PItem* items;
    const PScan* scans;
    float* aslots;                 // [slots][H][16 KB] block states
    float* pslots;                 // [slots][H][16 KB] inclusive prefixes (one launch)
    uint64_t* flags;               // [H][slots] (one launch): a head's flags contiguous
    int* hdr;                      // workspace header
    float* final_state;
    const float* ext_state;
    uint16_t* out;
    int H;
    int n_work;                    // workgroups of the launch (items x H)
    int n_flags;                   // slots x H
    int n_slots;                   // slots
    int plan_hash;
    int spin_limit;
    int force_timeout;
    int ordered;                   // one launch: take tickets (the launch may not fit at once)
};

typedef f32x4 State[kTiles];       // tile t = vb * 4 + kb; lane 16g + c holds
                                   // S[16 kb + 4 g + j][16 vb + c], j = 0..3

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ void zero_state(State& s) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) s[t] = zero4();
}

// One state slot as a 16 KB buffer window; lane l's piece of tile t is the
// 16 bytes at (t * 64 + l) * 16.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const float* base, int slot, int H,
                                                           int h) {
    const char* p = reinterpret_cast<const char*>(base) +
                    (int64_t(slot) * H + h) * int64_t(kStateBytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, kStateBytes,
                                             0x00020000);
}
template <int AUX>
__device__ __forceinline__ f32x4 slot_load(__amdgpu_buffer_rsrc_t r, int t, int lane) {
    return __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, uint32_t((t * 64 + lane) * 16), 0, AUX));
}
template <int AUX>
__device__ __forceinline__ void slot_store(__amdgpu_buffer_rsrc_t r, int t, int lane, f32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r,
                                           uint32_t((t * 64 + lane) * 16), 0, AUX);
}
template <int AUX>
__device__ __forceinline__ void store_state(const State& s, float* base, int slot, int H, int h,
                                            int lane) {
    const auto r = slot_rsrc(base, slot, H, h);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) slot_store<AUX>(r, t, lane, s[t]);
}

// Row-major [64][64] state (final_state / ext_state rows) <-> lane layout.
__device__ __forceinline__ void store_rows_state(const State& s, float* dst, int g, int c16) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const int kb = t & 3, vb = t >> 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[(16 * kb + 4 * g + j) * PD + 16 * vb + c16] = s[t][j];
    }
}
__device__ __forceinline__ f32x4 load_rows_tile(const float* src, int t, int g, int c16) {
    const int kb = t & 3, vb = t >> 2;
    f32x4 x;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = src[(16 * kb + 4 * g + j) * PD + 16 * vb + c16];
    return x;
}

// Device-coherent flag accesses (sc1), as the single-pass scans of the ROCm
// primitives library do on gfx942 / gfx950.
__device__ __forceinline__ uint64_t flag_load(const uint64_t* f) {
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(uint64_t* f, uint64_t x) {
    __hip_atomic_store(f, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Everything this wave stored has reached the coherence point, and no later
// memory operation is moved above this point by the compiler.
__device__ __forceinline__ void drain_stores() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
}
__device__ __forceinline__ void order_after_flag() {
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Flags carry the XCD of the workgroup that published (bits 8..11).  The
// XCDs' L2 caches are not coherent with each other, so a state published
// from another XCD is read with device-coherent loads (sc1, from memory); a
// state published from the reader's own XCD went through that XCD's L2 with
// the publisher's stores, so it is read there (sc0: past the CU's L1, which
// holds no line of it).  The kernel's workgroups of one head run on one XCD
// when the launch maps them there, which keeps most look-back reads in L2.
__device__ __forceinline__ uint64_t* flag_ptr(const PArgs& a, int slot, int h) {
    return a.flags + int64_t(h) * a.n_slots + slot;
}
__device__ __forceinline__ uint64_t xcd_tag() {
    return uint64_t(__builtin_amdgcn_s_getreg(kHwRegXccId) & 15) << 8;
}
__device__ __forceinline__ bool is_flag(uint64_t f, uint64_t kind) {
    return (f & ~kFlagXcd) == kind;
}

// Bounded wait for one flag to say "inclusive prefix published"; returns
// whether the publisher ran on this XCD (tag).  On timeout records
// LA_ERR_TIMEOUT and returns false (the caller carries on with whatever the
// slot holds: in bounds, not valid).
__device__ bool wait_prefix(const PArgs& a, const uint64_t* f, uint64_t tag) {
    uint64_t x = 0;
    for (int it = 0;; ++it) {
        x = a.force_timeout ? 0 : flag_load(f);
        if (is_flag(x, kFlagP)) break;
        if (it >= a.spin_limit) {
            __hip_atomic_fetch_or(a.hdr + piece::kStatusWord, LA_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
            x = 0;
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    order_after_flag();
    return __builtin_amdgcn_readfirstlane(int(is_flag(x, kFlagP) && (x & kFlagXcd) == tag)) != 0;
}

// A workgroup that is done with the flags (its waits are over and its
// states are published) is counted out by one of its waves -- the only wave
// of the workgroup that stores flags, or any wave when none does -- which
// first waits for its own stores.  The last workgroup counted clears the
// flags and the counters for the next pass: every reader of a flag has been
// counted before it, so no wait can see the clearing.
__device__ void retire(const PArgs& a, int lane) {
    drain_stores();
    int r = 0;
    if (lane == 0)
        r = __hip_atomic_fetch_add(a.hdr + piece::kRetireWord, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    if (__builtin_amdgcn_readfirstlane(r) == a.n_work - 1) {
        for (int i = lane; i < a.n_flags; i += 64) flag_store(a.flags + i, 0);
        if (lane == 0) {
            __hip_atomic_store(a.hdr + piece::kTicketWord, 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.hdr + piece::kRetireWord, 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The look-back of block j of a segment (slots slot0 .. slot0 + j - 1 hold
// its predecessors): the nearest predecessor m that has published its
// inclusive prefix, with every predecessor after it having published at
// least its aggregate.  The flags of up to 64 predecessors are polled at
// once, one per lane (lane i: predecessor j - 1 - i).  Block 0 of a segment
// always publishes its prefix, so the walk ends.  `local` tells whether
// every state the caller will read (the prefix and the aggregates after it)
// was published from this XCD (tag).  On timeout records LA_ERR_TIMEOUT and
// returns 0.
__device__ int find_prefix(const PArgs& a, int slot0, int j, int h, int lane, uint64_t tag,
                           bool& local) {
    bool passed_local = true;   // windows walked past: all their aggregates are read
    for (int base = j - 1;; base -= 64) {
        const int m = base - lane;
        for (int it = 0;; ++it) {
            const uint64_t f = (m >= 0 && !a.force_timeout)
                                   ? flag_load(flag_ptr(a, slot0 + m, h))
                                   : 0;
            const uint64_t bp = __builtin_amdgcn_ballot_w64(m >= 0 && is_flag(f, kFlagP));
            const uint64_t br = __builtin_amdgcn_ballot_w64(m < 0 || is_flag(f, kFlagP) ||
                                                            is_flag(f, kFlagA));
            const uint64_t bl = __builtin_amdgcn_ballot_w64(m < 0 || (f & kFlagXcd) == tag);
            if (bp) {
                const int l = __builtin_ctzll(bp);                 // nearest prefix
                const uint64_t need = l == 63 ? ~0ull : ((2ull << l) - 1);
                if ((br & need) == need) {
                    order_after_flag();
                    local = passed_local && (bl & need) == need;
                    return base - l;
                }
            } else if (br == ~0ull && base >= 64) {
                passed_local = passed_local && bl == ~0ull;
                break;                                             // next window
            }
            if (it >= a.spin_limit) {
                __hip_atomic_fetch_or(a.hdr + piece::kStatusWord, LA_ERR_TIMEOUT,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                order_after_flag();
                local = false;
                return 0;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
}

// ---------------------------------------------------------------------------
// Chunk data of one wave: k and v rows as loaded (64 tokens x 64 features
// each; load i gives lane l token 8 i + l / 8, features 8 (l % 8) .. + 7).
// ---------------------------------------------------------------------------
struct ChunkKV {
    u32x4 k[8], v[8];
};

__device__ __forceinline__ void load_chunk_kv(ChunkKV& r, const PArgs& a, int64_t tok0, int rows,
                                              int h, int lane) {
    const int64_t first = tok0 * a.H * PD;
    const auto rk = chunk_rsrc(a.k, first, 2, rows, a.H, PD);
    const auto rv = chunk_rsrc(a.v, first, 2, rows, a.H, PD);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t off = uint32_t((((8 * i + (lane >> 3)) * a.H + h) * PD + 8 * (lane & 7)) * 2);
        r.k[i] = buf_load16(rk, off);
        r.v[i] = buf_load16(rv, off);
    }
}

// The inverse: slot order (features 4 g .. and 16 + 4 g .. of a 32-feature
// half) back to 16 contiguous bytes (features 8 g .. + 7).
__device__ __forceinline__ u32x4 from_slot_order(u32x4 x) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
    const auto r0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
    const auto r1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
    return u32x4{r0[0], r1[0], r0[1], r1[1]};
}

// Registers -> the wave's LDS tiles, row-major (160-byte rows).
__device__ __forceinline__ void stage_chunk(const ChunkKV& r, uint16_t* sK, uint16_t* sV,
                                            int lane) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int o = (8 * i + (lane >> 3)) * PLD + 8 * (lane & 7);
        *reinterpret_cast<u32x4*>(sK + o) = r.k[i];
        *reinterpret_cast<u32x4*>(sV + o) = r.v[i];
    }
    // the wave reads what it wrote: LDS operations of one wave complete in
    // order, the wait keeps the compiler from moving the reads up
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_wave_barrier();
}

// S += K^T V of the staged chunk (accumulator tile (kb, vb)).
__device__ __forceinline__ void acc_kv(State& S, const uint16_t* sK, const uint16_t* sV, int g,
                                       int c16) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        u32x4 ak[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ak[i] = tr_frag(sK, PLD, 16 * i, ks, g, c16);
            bv[i] = tr_frag(sV, PLD, 16 * i, ks, g, c16);
        }
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                S[vb * 4 + kb] = mfma_bf16(ak[kb], bv[vb], S[vb * 4 + kb]);
    }
}

// Outputs of a piece are built in two parts.  The part within the piece,
//   O_c = tril(Q_c K_c^T) V_c               (each chunk c),
//   O_1 += (Q_1 K_0^T) V_0                   (chunk 1 sees all of chunk 0),
// needs nothing but the piece's own q, k and v, so it is computed while the
// workgroups before it publish their states.  The state the piece starts
// from, S = S_b + E_p (the block's starting state plus the pieces before it
// in the block), enters once the look-back has S_b: O_c += Q_c S.  O^T is kept
// in fp32 MFMA accumulators: tile tb * 4 + fb, lane 16 g + c: token 16 tb + c,
// features 16 fb + 4 g .. + 3; written as bf16 (round to nearest even).  The
// scores P = Q K^T of a chunk and across the two chunks enter their products
// as bf16 (round to nearest even), the state as two bf16 terms.
typedef f32x4 OTiles[16];

// q of a chunk as the B operand of the products over d_k, in k-slot order:
// lane 16 g + c holds token 16 tb + c; in a K = 32 step ks, features
// 32 ks + 4 g .. + 3 (elements 0..3) and 32 ks + 16 + 4 g .. + 3 (elements
// 4..7) -- the order in which a state's accumulator tiles (kb = 2 ks,
// 2 ks + 1) hold their rows, so a state feeds the products straight from
// registers.  Loaded as two 8-byte pieces per step.
struct QSlots {
    u32x4 q[4][2];
};
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ void load_q_slots(QSlots& qs, const PArgs& a, int64_t tok0, int rows,
                                             int h, int g, int c16) {
    const auto rq = chunk_rsrc(a.q, tok0 * a.H * PD, 2, rows, a.H, PD);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint32_t off =
                uint32_t((((16 * tb + c16) * a.H + h) * PD + 32 * ks + 4 * g) * 2);
            const u32x2 x = buf_load8(rq, off), y = buf_load8(rq, off + 32);
            qs.q[tb][ks] = u32x4{x[0], x[1], y[0], y[1]};
        }
}

// S^T as A operands, split into two bf16 terms S = hi + lo (the split keeps
// the fp32 state's precision in the bf16 product).
struct SSplit {
    u32x4 hi[4][2], lo[4][2];
};
__device__ __forceinline__ void split_state(const State& S, SSplit& sp) {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const f32x4 x = S[fb * 4 + 2 * ks], y = S[fb * 4 + 2 * ks + 1];
            const uint32_t h0 = cvt_bf2(x[0], x[1]), h1 = cvt_bf2(x[2], x[3]);
            const uint32_t h2 = cvt_bf2(y[0], y[1]), h3 = cvt_bf2(y[2], y[3]);
            sp.hi[fb][ks] = u32x4{h0, h1, h2, h3};
            sp.lo[fb][ks] = u32x4{cvt_bf2(x[0] - bf_lo(h0), x[1] - bf_hi(h0)),
                                  cvt_bf2(x[2] - bf_lo(h1), x[3] - bf_hi(h1)),
                                  cvt_bf2(y[0] - bf_lo(h2), y[1] - bf_hi(h2)),
                                  cvt_bf2(y[2] - bf_lo(h3), y[3] - bf_hi(h3))};
        }
}

// O += Q S for the chunk's 64 tokens (both terms of S, hi first).
__device__ __forceinline__ void add_qs(OTiles& O, const SSplit& sp, const QSlots& qs) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                O[tb * 4 + fb] = mfma_bf16(sp.hi[fb][ks], qs.q[tb][ks], O[tb * 4 + fb]);
                O[tb * 4 + fb] = mfma_bf16(sp.lo[fb][ks], qs.q[tb][ks], O[tb * 4 + fb]);
            }
}

// Scores of 16 queries (slot-order q, B operand) against the 4 key tiles
// of a chunk (K rows in slot order, A operands) -> P^T as bf16 B operands of
// the value product: pb[pp] covers key tiles 2 pp, 2 pp + 1.  Key tiles past
// NK - 1 are not computed (zero); with DIAG the last one is masked causally
// (key u <= query t).
template <int NK, bool DIAG>
__device__ __forceinline__ void score_tiles(u32x4 (&pb)[2], const u32x4 (&kr)[4][2],
                                            const u32x4 (&qt)[2], int g, int c16) {
    f32x4 p[NK];
#pragma unroll
    for (int ub = 0; ub < NK; ++ub) {
        p[ub] = mfma_bf16(kr[ub][0], qt[0], zero4());
        p[ub] = mfma_bf16(kr[ub][1], qt[1], p[ub]);
    }
    if constexpr (DIAG) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (4 * g + j > c16) p[NK - 1][j] = 0.f;
    }
#pragma unroll
    for (int pp = 0; pp < (NK + 1) / 2; ++pp) {
        const f32x4 x = p[2 * pp];
        const f32x4 y = 2 * pp + 1 < NK ? p[2 * pp + 1] : zero4();
        pb[pp] = u32x4{cvt_bf2(x[0], x[1]), cvt_bf2(x[2], x[3]), cvt_bf2(y[0], y[1]),
                       cvt_bf2(y[2], y[3])};
    }
}

// O (tokens 16 TB ..) = tril(Q K^T) V within the staged chunk.
template <int TB>
__device__ __forceinline__ void intra_tokens(OTiles& O, const u32x4 (&kr)[4][2],
                                             const u32x4 (&vt)[4][2], const u32x4 (&qt)[2],
                                             int g, int c16) {
    u32x4 pb[2];
    score_tiles<TB + 1, true>(pb, kr, qt, g, c16);
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
        f32x4 o = zero4();
#pragma unroll
        for (int pp = 0; pp <= TB / 2; ++pp) o = mfma_bf16(vt[fb][pp], pb[pp], o);
        O[TB * 4 + fb] = o;
    }
}

// O (tokens 16 TB .. of chunk 1) += (Q_1 K_0^T) V_0: every key of chunk 0.
template <int TB>
__device__ __forceinline__ void cross_tokens(OTiles& O, const u32x4 (&kr0)[4][2],
                                             const u32x4 (&vt0)[4][2], const u32x4 (&qt)[2],
                                             int g, int c16) {
    u32x4 pb[2];
    score_tiles<4, false>(pb, kr0, qt, g, c16);
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
        O[TB * 4 + fb] = mfma_bf16(vt0[fb][0], pb[0], O[TB * 4 + fb]);
        O[TB * 4 + fb] = mfma_bf16(vt0[fb][1], pb[1], O[TB * 4 + fb]);
    }
}

// K rows in slot order (two 8-byte reads) and V^T fragments in token order
// of the staged chunk: the operands of its score and value products.
__device__ __forceinline__ void chunk_operands(u32x4 (&kr)[4][2], u32x4 (&vt)[4][2],
                                               const uint16_t* sK, const uint16_t* sV, int g,
                                               int c16) {
#pragma unroll
    for (int ub = 0; ub < 4; ++ub)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint16_t* p = sK + (16 * ub + c16) * PLD + 32 * ks + 4 * g;
            kr[ub][ks] = cat2(lds_u32x2(p), lds_u32x2(p + 16));
            vt[ub][ks] = tr_frag(sV, PLD, 16 * ub, ks, g, c16);
        }
}

// O = tril(Q K^T) V of the staged chunk; its operands are left in kr, vt.
__device__ __forceinline__ void chunk_intra(OTiles& O, u32x4 (&kr)[4][2], u32x4 (&vt)[4][2],
                                            const uint16_t* sK, const uint16_t* sV,
                                            const QSlots& qs, int g, int c16) {
    chunk_operands(kr, vt, sK, sV, g, c16);
    intra_tokens<0>(O, kr, vt, qs.q[0], g, c16);
    intra_tokens<1>(O, kr, vt, qs.q[1], g, c16);
    intra_tokens<2>(O, kr, vt, qs.q[2], g, c16);
    intra_tokens<3>(O, kr, vt, qs.q[3], g, c16);
}
__device__ __forceinline__ void chunk_cross(OTiles& O, const u32x4 (&kr0)[4][2],
                                            const u32x4 (&vt0)[4][2], const QSlots& qs, int g,
                                            int c16) {
    cross_tokens<0>(O, kr0, vt0, qs.q[0], g, c16);
    cross_tokens<1>(O, kr0, vt0, qs.q[1], g, c16);
    cross_tokens<2>(O, kr0, vt0, qs.q[2], g, c16);
    cross_tokens<3>(O, kr0, vt0, qs.q[3], g, c16);
}

// Rows tok0 .. tok0 + rows - 1 of out from O (rows past `rows` fall outside
// the buffer window).  Lane (g, c16) holds 16 contiguous bytes of token
// 16 tb + c16 in each feature half hh (features 32 hh + 8 g ..); neighbouring
// tokens' lanes (c16, c16 ^ 1) swap one piece, so that each store writes
// whole 128-byte rows (8 lanes per token): the even tokens' rows, then the
// odd tokens'.  The outputs are nontemporal stores, which go to memory as
// they are written: whole rows make whole lines.
__device__ __forceinline__ void store_chunk(const OTiles& O, const PArgs& a, int64_t tok0,
                                            int rows, int h, int g, int c16) {
    const auto ro = chunk_rsrc(a.out, tok0 * a.H * PD, 2, rows, a.H, PD);
    const bool odd = (c16 & 1) != 0;
    const uint32_t row_bytes = uint32_t(a.H * PD * 2);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        u32x4 pc[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const f32x4 x = O[tb * 4 + 2 * hh], y = O[tb * 4 + 2 * hh + 1];
            pc[hh] = from_slot_order(u32x4{cvt_bf2(x[0], x[1]), cvt_bf2(x[2], x[3]),
                                           cvt_bf2(y[0], y[1]), cvt_bf2(y[2], y[3])});
        }
        const u32x4 give = odd ? pc[0] : pc[1];
        u32x4 got;
#pragma unroll
        for (int i = 0; i < 4; ++i)   // quad_perm [1, 0, 3, 2]: lane c16 ^ 1
            got[i] = __builtin_amdgcn_mov_dpp(int(give[i]), 0xB1, 0xF, 0xF, false);
        // lane's own token row and feature-half offsets
        const uint32_t own = uint32_t(((16 * tb + c16) * a.H + h) * PD * 2) + 16 * g;
        // even token rows: even lanes their half 0, odd lanes the even token's half 1
        buf_store16u(ro, odd ? own - row_bytes + 64 : own, odd ? got : pc[0]);
        // odd token rows: even lanes the odd token's half 0, odd lanes their half 1
        buf_store16u(ro, odd ? own + 64 : own + row_bytes, odd ? pc[1] : got);
    }
}

// The part of one wave's piece (up to two chunks) within the piece: O0, O1.
// Chunk 0's k / v are staged on entry; chunk 1's are in r1 (`same` false:
// chunk 1 belongs to another branch and sees nothing of chunk 0).
__device__ __forceinline__ void piece_intra(OTiles& O0, OTiles& O1, uint16_t* sK, uint16_t* sV,
                                            const ChunkKV& r1, const QSlots& qs0,
                                            const QSlots& qs1, int n0, int n1, bool same, int g,
                                            int c16, int lane) {
    if (n0 <= 0) return;
    u32x4 kr0[4][2], vt0[4][2];
    chunk_intra(O0, kr0, vt0, sK, sV, qs0, g, c16);
    if (n1 > 0) {
        // every lane's reads of chunk 0 are done before chunk 1 overwrites it
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
        stage_chunk(r1, sK, sV, lane);
        {
            u32x4 kr1[4][2], vt1[4][2];
            chunk_intra(O1, kr1, vt1, sK, sV, qs1, g, c16);
        }
        if (same) chunk_cross(O1, kr0, vt0, qs1, g, c16);
    }
}

// ---------------------------------------------------------------------------
// State sums split over the four waves: wave w adds tiles 4 w .. 4 w + 3.
// ---------------------------------------------------------------------------
// acc += slot tiles of slots first .. first + n - 1, in order.  Loads go out
// in batches of four slots with the next batch issued before the current one
// is added, so two batches are in flight.
template <int AUX>
__device__ __forceinline__ void add_slots4(f32x4 (&acc)[4], const float* base, int first, int n,
                                           int H, int h, int w, int lane) {
    // batch of 4 slots from s0; slots past n read an empty window (zeros,
    // no memory access)
    auto load4 = [&](f32x4 (&x)[4][4], int s0) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const auto r = s0 + b < n ? slot_rsrc(base, first + s0 + b, H, h)
                                      : __builtin_amdgcn_make_buffer_rsrc(
                                            const_cast<float*>(base), (short)0, 0, 0x00020000);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[b][i] = slot_load<AUX>(r, 4 * w + i, lane);
        }
    };
    auto add4 = [&](const f32x4 (&x)[4][4], int s0) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (s0 + b < n)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += x[b][i];
    };
    if (n <= 0) return;
    // two batches in flight, alternating buffers: each add waits only for
    // its own batch (loads complete in order), while the next is loading
    f32x4 xa[4][4], xb[4][4];
    load4(xa, 0);
    for (int s0 = 0; s0 < n; s0 += 8) {
        load4(xb, s0 + 4);
        add4(xa, s0);
        load4(xa, s0 + 8);
        add4(xb, s0 + 4);
    }
}

// own = P_m + A_{m+1} + ... + A_{j-1} (this wave's four tiles), read with
// cache policy AUX.
template <int AUX>
__device__ __forceinline__ void look_back(f32x4 (&own)[4], const PArgs& a, int slot0, int m,
                                          int j, int h, int w, int lane) {
    const auto r = slot_rsrc(a.pslots, slot0 + m, a.H, h);
#pragma unroll
    for (int i = 0; i < 4; ++i) own[i] = slot_load<AUX>(r, 4 * w + i, lane);
    add_slots4<AUX>(own, a.aslots, slot0 + m + 1, j - 1 - m, a.H, h, w, lane);
}

// LDS exchange region: two states in the lane layout.
struct Xch {
    f32x4 x[2][kTiles * 64];
};
__device__ __forceinline__ void put_state(Xch& X, int b, const State& s, int lane) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) X.x[b][t * 64 + lane] = s[t];
}
__device__ __forceinline__ void get_state(const Xch& X, int b, State& s, int lane) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) s[t] = X.x[b][t * 64 + lane];
}
__device__ __forceinline__ void put_tiles4(Xch& X, int b, const f32x4 (&v)[4], int w, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) X.x[b][(4 * w + i) * 64 + lane] = v[i];
}

// The state a branch starts from (whole, in the lane layout): its view's
// total (seed >= 0: the view's scan entry), ext_state row -seed - 2
// (seed <= -2), or zero (seed == -1).  In the single-launch form the view's
// inclusive prefix is awaited; in the three-launch form the prefix launch
// left it in the view's last slot; in the two-launch form the view's block
// states are summed from zero, in slot order.
template <int MODE>
__device__ __forceinline__ void load_seed(State& S, const PArgs& a, int seed, int h, int g,
                                          int c16, int lane) {
    const int H = a.H;
    zero_state(S);
    if (seed >= 0) {
        const PScan vs = a.scans[seed];
        const int last = vs.first_slot + vs.n_slots - 1;
        if constexpr (MODE == kFused) {
            const auto r = slot_rsrc(a.pslots, last, H, h);
            if (wait_prefix(a, flag_ptr(a, last, h), xcd_tag())) {
#pragma unroll
                for (int t = 0; t < kTiles; ++t) S[t] = slot_load<kAuxL2>(r, t, lane);
            } else {
#pragma unroll
                for (int t = 0; t < kTiles; ++t) S[t] = slot_load<kAuxCoherent>(r, t, lane);
            }
        } else if constexpr (MODE == kOut3) {
            const auto r = slot_rsrc(a.aslots, last, H, h);
#pragma unroll
            for (int t = 0; t < kTiles; ++t) S[t] = slot_load<0>(r, t, lane);
        } else {
            for (int s = 0; s < vs.n_slots; ++s) {
                const auto r = slot_rsrc(a.aslots, vs.first_slot + s, H, h);
#pragma unroll
                for (int t = 0; t < kTiles; ++t) S[t] += slot_load<0>(r, t, lane);
            }
        }
    } else if (seed <= -2) {
        const float* src = a.ext_state + (int64_t(-seed - 2) * H + h) * PD * PD;
#pragma unroll
        for (int t = 0; t < kTiles; ++t) S[t] = load_rows_tile(src, t, g, c16);
    }
}

// ---------------------------------------------------------------------------
// The kernel (all forms).
// ---------------------------------------------------------------------------
template <int MODE>
// The first arguments repeat what the kernel reads before its first load,
// so that they arrive in registers (kernel argument preloading) rather than
// through a load of the argument block.
__global__ __launch_bounds__(kThreads) void piece_kernel(const int32_t* plan, const PItem* items,
                                                         int n_work, int H_, int plan_hash,
                                                         int ordered, PArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sStage[4][2][kStageElems];
    __shared__ Xch X;
    __shared__ int sB[2];
    const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    uint16_t* sK = sStage[w][0];
    uint16_t* sV = sStage[w][1];
    const int H = a.H;

    // In index mode the work's item is known at once: its record (inside
    // the plan's info->plan_words words) is read together with the plan
    // check, and nothing of it is used unless the check passes.
    int work = blockIdx.x;
    const bool by_index = !(MODE == kFused && ordered);
    PItemBlock ib = reinterpret_cast<const PItemBlock*>(
        items)[by_index ? min(work, n_work - 1) / H_ : 0];   // n_work >= 1

    // the plan must be the one the pass info was built with (both words are
    // read before either is tested, and the item's with them: the empty asm
    // takes the item's words, so their loads are not moved past the test)
    const int magic = plan[0], hash = plan[LA_PLAN_HASH_WORD];
    asm volatile("" ::"s"(ib.kind), "s"(ib.n), "s"(ib.b0), "s"(ib.unused), "s"(ib.blk.tok0),
                 "s"(ib.blk.ntok), "s"(ib.blk.slot), "s"(ib.blk.seed), "s"(ib.blk.seg),
                 "s"(ib.blk.slot0), "s"(ib.blk.j), "s"(ib.blk.final_row), "s"(magic), "s"(hash));
    if ((magic != LA_PLAN_MAGIC) | (hash != plan_hash)) {
        if (tid == 0)
            __hip_atomic_fetch_or(a.hdr + piece::kStatusWord, LA_ERR_PLAN, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    if (!by_index) {
        // tickets in launch order of the items: everything a workgroup waits
        // for belongs to a smaller ticket, held by a running workgroup.  (When
        // every workgroup of the launch is resident at once, waits need no
        // order and the index is the work.)
        if (tid == 0)
            sB[0] = __hip_atomic_fetch_add(a.hdr + piece::kTicketWord, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        work = sB[0];
        if (work < a.n_work)
            ib = reinterpret_cast<const PItemBlock*>(
                a.items)[__builtin_amdgcn_readfirstlane(work / H)];
    }
    if (work < a.n_work) {
        const int h = work % H;
        if (ib.kind == LA_ITEM_BLOCK) {
            const PBlock B = ib.blk;
            const int np = (B.ntok + 2 * kChunk - 1) / (2 * kChunk);   // pieces
            const int64_t ptok0 = int64_t(B.tok0) + w * 2 * kChunk;
            const int pntok = min(2 * kChunk, B.ntok - w * 2 * kChunk);   // <= 0: no piece
            ChunkKV r0, r1;
            QSlots qs0, qs1;
            load_chunk_kv(r0, a, ptok0, pntok, h, lane);
            load_chunk_kv(r1, a, ptok0 + kChunk, pntok - kChunk, h, lane);

            // the piece's own state, chunk 1 first so chunk 0 stays staged
            State A;
            zero_state(A);
            if (pntok > kChunk) {
                stage_chunk(r1, sK, sV, lane);
                acc_kv(A, sK, sV, g, c16);
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                __builtin_amdgcn_wave_barrier();
            }
            if (pntok > 0) {
                stage_chunk(r0, sK, sV, lane);
                acc_kv(A, sK, sV, g, c16);
            }

            // q is loaded once k and v are in (they come first: every block
            // after this one waits for the state they give).  The wave that
            // publishes the block's state loads its q after the publication:
            // the wait before the flag covers every load the wave has in
            // flight, q included
            __builtin_amdgcn_sched_barrier(0);
            const bool publisher = MODE == kFused && B.slot >= 0 && w == np - 1;
            if constexpr (MODE != kStates) {
                if (!publisher) {
                    load_q_slots(qs0, a, ptok0, pntok, h, g, c16);
                    load_q_slots(qs1, a, ptok0 + kChunk, pntok - kChunk, h, g, c16);
                }
            }
            // in-block prefix over the pieces: E_w and A_b (wave np - 1)
            State E, Ab;
            zero_state(E);
            if (w == 0 && np > 1) put_state(X, 0, A, lane);
            if (w == 2 && np > 3) put_state(X, 1, A, lane);
            __syncthreads();
            State T;
            if (w == 1 && np > 1) {
                State x;
                get_state(X, 0, x, lane);
#pragma unroll
                for (int t = 0; t < kTiles; ++t) E[t] = zero4() + x[t];
                if (np > 2) {
                    State i1;
#pragma unroll
                    for (int t = 0; t < kTiles; ++t) i1[t] = E[t] + A[t];
                    put_state(X, 0, i1, lane);
                }
            }
            if (w == 3 && np > 3) get_state(X, 1, T, lane);
            __syncthreads();
            if ((w == 2 && np > 2) || (w == 3 && np > 3)) get_state(X, 0, E, lane);
            if (w == 3 && np > 3) {
#pragma unroll
                for (int t = 0; t < kTiles; ++t) E[t] = E[t] + T[t];
            }
            if (w == np - 1) {
#pragma unroll
                for (int t = 0; t < kTiles; ++t) Ab[t] = (w == 0 ? zero4() : E[t]) + A[t];
            }
            __syncthreads();   // X is reused below

            if constexpr (MODE == kStates) {
                if (w == np - 1 && B.slot >= 0) store_state<0>(Ab, a.aslots, B.slot, H, h, lane);
            } else {
                // own: the segment's state before this block (fold of the
                // earlier blocks' states), seed: where a branch starts
                const bool has_seed = B.seed != -1;
                f32x4 own4[4], sin4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) own4[i] = zero4();
                if constexpr (MODE == kFused) {
                    if (B.slot >= 0 && w == np - 1) {
                        if (B.j == 0) {
                            State P;
#pragma unroll
                            for (int t = 0; t < kTiles; ++t) P[t] = zero4() + Ab[t];
                            store_state<kAuxCoherent>(P, a.pslots, B.slot, H, h, lane);
                            drain_stores();
                            if (lane == 0)
                                flag_store(flag_ptr(a, B.slot, h), kFlagP | xcd_tag());
                        } else {
                            store_state<kAuxCoherent>(Ab, a.aslots, B.slot, H, h, lane);
                            drain_stores();
                            if (lane == 0)
                                flag_store(flag_ptr(a, B.slot, h), kFlagA | xcd_tag());
                        }
                    }
                }
                if (publisher) {
                    load_q_slots(qs0, a, ptok0, pntok, h, g, c16);
                    load_q_slots(qs1, a, ptok0 + kChunk, pntok - kChunk, h, g, c16);
                }
                // the part of the outputs within each piece, computed while
                // the blocks before finish publishing
                OTiles O0, O1;
                piece_intra(O0, O1, sK, sV, r1, qs0, qs1, pntok, pntok - kChunk, true, g, c16,
                            lane);
                if constexpr (MODE == kFused) {
                    if (B.j > 0) {
                        // nearest predecessor with an inclusive prefix, then
                        // the aggregates after it, left to right
                        bool local;
                        const int m = find_prefix(a, B.slot0, B.j, h, lane, xcd_tag(), local);
                        if (__builtin_amdgcn_readfirstlane(int(local)))
                            look_back<kAuxL2>(own4, a, B.slot0, m, B.j, h, w, lane);
                        else
                            look_back<kAuxCoherent>(own4, a, B.slot0, m, B.j, h, w, lane);
                    }
                } else if (B.j > 0) {
                    if constexpr (MODE == kOut3) {
                        const auto r = slot_rsrc(a.aslots, B.slot0 + B.j - 1, H, h);
#pragma unroll
                        for (int i = 0; i < 4; ++i) own4[i] = slot_load<0>(r, 4 * w + i, lane);
                    } else {
                        add_slots4<0>(own4, a.aslots, B.slot0, B.j, H, h, w, lane);
                    }
                }
                // seed tiles of this wave
#pragma unroll
                for (int i = 0; i < 4; ++i) sin4[i] = zero4();
                if (B.seed >= 0) {
                    const PScan vs = a.scans[B.seed];
                    const int last = vs.first_slot + vs.n_slots - 1;
                    if (MODE == kFused && !a.ordered) {
                        // every block of the view is running: sum its
                        // states here rather than wait for its last block
                        bool local;
                        const int m = find_prefix(a, vs.first_slot, vs.n_slots, h, lane, xcd_tag(),
                                                  local);
                        if (__builtin_amdgcn_readfirstlane(int(local)))
                            look_back<kAuxL2>(sin4, a, vs.first_slot, m, vs.n_slots, h, w, lane);
                        else
                            look_back<kAuxCoherent>(sin4, a, vs.first_slot, m, vs.n_slots, h, w,
                                                    lane);
                    } else if constexpr (MODE == kFused) {
                        const auto r = slot_rsrc(a.pslots, last, H, h);
                        if (wait_prefix(a, flag_ptr(a, last, h), xcd_tag())) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                sin4[i] = slot_load<kAuxL2>(r, 4 * w + i, lane);
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                sin4[i] = slot_load<kAuxCoherent>(r, 4 * w + i, lane);
                        }
                    } else if constexpr (MODE == kOut3) {
                        const auto r = slot_rsrc(a.aslots, last, H, h);
#pragma unroll
                        for (int i = 0; i < 4; ++i) sin4[i] = slot_load<0>(r, 4 * w + i, lane);
                    } else {
                        add_slots4<0>(sin4, a.aslots, vs.first_slot, vs.n_slots, H, h, w, lane);
                    }
                } else if (B.seed <= -2) {
                    const float* src = a.ext_state + (int64_t(-B.seed - 2) * H + h) * PD * PD;
#pragma unroll
                    for (int i = 0; i < 4; ++i) sin4[i] = load_rows_tile(src, 4 * w + i, g, c16);
                }
                // S_b = seed (or 0), += own if the block has predecessors
                if (B.j > 0)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sin4[i] += own4[i];
                put_tiles4(X, 0, own4, w, lane);
                put_tiles4(X, 1, sin4, w, lane);
                __syncthreads();
                // the block's inclusive prefix, where it is needed: a view's
                // total (final_state), and the prefix later look-backs use
                // when the work comes by ticket
                const bool need_p = B.final_row >= 0 ||
                                    (MODE == kFused && a.ordered && B.slot >= 0 && B.j > 0);
                if (w == np - 1 && need_p && (MODE == kFused || MODE == kOut2)) {
                    // own + A_b.  A_b is read back from its slot (this wave
                    // published it in one launch; the states launch wrote it
                    // in the two-launch form), which frees its registers for
                    // the products
                    State P;
                    {
                        const float* ab = MODE == kFused && B.j == 0 ? a.pslots : a.aslots;
                        const auto r = slot_rsrc(ab, B.slot, H, h);
#pragma unroll
                        for (int t = 0; t < kTiles; ++t) P[t] = slot_load<kAuxL2>(r, t, lane);
                    }
                    if (B.j > 0) {
                        State own;
                        get_state(X, 0, own, lane);
#pragma unroll
                        for (int t = 0; t < kTiles; ++t) P[t] = own[t] + P[t];
                    } else {
#pragma unroll
                        for (int t = 0; t < kTiles; ++t) P[t] = zero4() + P[t];
                    }
                    // published where a look-back can use it: a view's total
                    // (branches' seed), and every block when the work comes by
                    // ticket (later blocks may start after this one ends); when
                    // the whole grid runs at once every look-back runs while
                    // its predecessors' prefixes are still being formed, and
                    // finds its segment's first block
                    if (MODE == kFused && B.slot >= 0 && B.j > 0 &&
                        (a.ordered || B.final_row >= 0)) {
                        store_state<kAuxCoherent>(P, a.pslots, B.slot, H, h, lane);
                        drain_stores();
                        if (lane == 0)
                            flag_store(flag_ptr(a, B.slot, h), kFlagP | xcd_tag());
                    }
                    if (B.final_row >= 0)
                        store_rows_state(P, a.final_state + (int64_t(B.final_row) * H + h) * PD * PD,
                                         g, c16);
                }
                // the flags are done with: the publishing wave counts the
                // workgroup out before its outputs
                if (MODE == kFused && w == np - 1) retire(a, lane);
                // O += Q S, S = S_b + E_p: the block's starting state and the
                // pieces before this one in the block
                if (pntok > 0 && (has_seed || B.j > 0 || w >= 1)) {
                    SSplit sp;
                    {
                        State S;
                        get_state(X, 1, S, lane);
                        if (!has_seed && B.j == 0) zero_state(S);
                        if (w >= 1)
#pragma unroll
                            for (int t = 0; t < kTiles; ++t) S[t] = S[t] + E[t];
                        split_state(S, sp);
                    }
                    add_qs(O0, sp, qs0);
                    if (pntok > kChunk) add_qs(O1, sp, qs1);
                }
                if (pntok > 0) store_chunk(O0, a, ptok0, min(pntok, kChunk), h, g, c16);
                if (pntok > kChunk) store_chunk(O1, a, ptok0 + kChunk, pntok - kChunk, h, g, c16);
            }
        } else if constexpr (MODE != kStates) {
            // packed branches: wave w takes block b_2w and, when there is one,
            // block b_2w+1 (then both are one chunk long), each from its seed
            const PItem it = __builtin_bit_cast(PItem, ib);
            // this wave's pair, selected (an index into the record would put
            // it on the stack)
            const int b0 = w == 0 ? it.b[0] : w == 1 ? it.b[2] : w == 2 ? it.b[4] : it.b[6];
            const int b1 = w == 0 ? it.b[1] : w == 1 ? it.b[3] : w == 2 ? it.b[5] : it.b[7];
            // when every branch of the pack starts from one view's total and
            // the whole grid is resident, the four waves sum the view's
            // states themselves (four tiles each) instead of waiting for the
            // view's last block to publish it
            int shared = -1;
            if (MODE == kFused && !a.ordered) {
                int sd = -1;
                bool same = true;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int b = it.b[i];
                    if (b >= 0) {
                        const int x = a.blocks[b].seed;
                        if (sd == -1) sd = x;
                        same = same && x == sd && x >= 0;
                    }
                }
                shared = same ? sd : -1;
            }
            const PBlock B = a.blocks[b0 >= 0 ? b0 : 0];
            const PBlock B1 = b1 >= 0 ? a.blocks[b1] : B;
            // chunk 1: the branch's second chunk, or the second branch
            const int64_t t1 = b1 >= 0 ? int64_t(B1.tok0) : int64_t(B.tok0) + kChunk;
            const int n1 = b1 >= 0 ? B1.ntok : B.ntok - kChunk;
            OTiles O0, O1;
            QSlots qs0, qs1;
            if (b0 >= 0) {
                ChunkKV r0, r1;
                load_chunk_kv(r0, a, B.tok0, B.ntok, h, lane);
                load_chunk_kv(r1, a, t1, n1, h, lane);
                load_q_slots(qs0, a, B.tok0, B.ntok, h, g, c16);
                load_q_slots(qs1, a, t1, n1, h, g, c16);
                // local parts first (a branch's own tokens, from a zero
                // state), then each branch's seed
                stage_chunk(r0, sK, sV, lane);
                piece_intra(O0, O1, sK, sV, r1, qs0, qs1, min(B.ntok, kChunk), n1, b1 < 0, g, c16,
                            lane);
            }
            if (shared >= 0) {
                const PScan vs = a.scans[shared];
                f32x4 tot4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) tot4[i] = zero4();
                bool local;
                const int m = find_prefix(a, vs.first_slot, vs.n_slots, h, lane, xcd_tag(), local);
                if (__builtin_amdgcn_readfirstlane(int(local)))
                    look_back<kAuxL2>(tot4, a, vs.first_slot, m, vs.n_slots, h, w, lane);
                else
                    look_back<kAuxCoherent>(tot4, a, vs.first_slot, m, vs.n_slots, h, w, lane);
                put_tiles4(X, 0, tot4, w, lane);
                __syncthreads();
                if (MODE == kFused && w == 0) retire(a, lane);
            }
            if (b0 >= 0) {
                SSplit sp;
                {
                    State Sb;
                    if (shared >= 0)
                        get_state(X, 0, Sb, lane);
                    else
                        load_seed<MODE>(Sb, a, B.seed, h, g, c16, lane);
                    split_state(Sb, sp);
                }
                add_qs(O0, sp, qs0);
                if (n1 > 0) {
                    if (b1 >= 0 && B1.seed != B.seed) {
                        State Sb;
                        load_seed<MODE>(Sb, a, B1.seed, h, g, c16, lane);
                        split_state(Sb, sp);
                    }
                    add_qs(O1, sp, qs1);
                }
                store_chunk(O0, a, B.tok0, min(B.ntok, kChunk), h, g, c16);
                if (n1 > 0) store_chunk(O1, a, t1, n1, h, g, c16);
            }
            if (MODE == kFused && shared < 0) {
                __syncthreads();   // every wave's seed wait is over
                if (w == 0) retire(a, lane);
            }
        }
    } else if (MODE == kFused && w == 0) {
        retire(a, lane);   // no work (not launched so: the grid is the work)
    }

}

// Layout of the piece path's part of a workspace (after the header).
struct WsLayout {
    size_t flags, aslots, pslots, total;
};
WsLayout ws_layout(const la_pass_info& info, int32_t H) {
    WsLayout l;
    const size_t nsh = size_t(info.piece_slots) * size_t(H);
    l.flags = piece::kHeaderBytes;
    l.aslots = (l.flags + nsh * sizeof(uint64_t) + 255) / 256 * 256;
    l.pslots = l.aslots + nsh * size_t(kStateBytes);
    l.total = l.pslots + nsh * size_t(kStateBytes);
    return l;
}

// Workgroups of the single-launch kernel the current device holds at once
// (0 when unknown).  A launch of at most that many workgroups is resident in
// full, so its waits need no ordering of the work.
int resident_capacity() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(piece_kernel<kFused>), kThreads, 0) !=
            hipSuccess)
        return 0;
    const int c = cus > 0 && per_cu > 0 ? cus * per_cu : 0;
    if (dev < 64 && c > 0) cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

}  // namespace

namespace piece {

size_t workspace_bytes(const la_pass_info& info, int32_t H) { return ws_layout(info, H).total; }

la_status launch(int32_t stages, int form, const void* q, const void* k, const void* v,
                 int32_t H, const la_pass_info& info, const int32_t* plan,
                 const float* ext_state, void* out, float* final_state, void* workspace,
                 hipStream_t st, int32_t spin_limit, bool force_timeout, bool ordered) {
    const WsLayout l = ws_layout(info, H);
    char* ws = static_cast<char*>(workspace);
    PArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    // table offsets from the pass info (the plan itself is device memory)
    const int64_t off_pblocks = int64_t(LA_PLAN_HEADER_WORDS) +
                                int64_t(info.n_blocks) * LA_PLAN_BLOCK_WORDS +
                                int64_t(info.n_delta) * LA_PLAN_DELTA_WORDS +
                                int64_t(info.n_scan) * LA_PLAN_SCAN_WORDS;
    const int64_t off_pitems = off_pblocks + int64_t(info.piece_blocks) * LA_PLAN_BLOCK_WORDS;
    const int64_t off_pscan = off_pitems + int64_t(info.piece_items) * LA_PLAN_ITEM_WORDS;
    a.plan = plan;
    a.blocks = reinterpret_cast<const PBlock*>(plan + off_pblocks);
    a.items = reinterpret_cast<const PItem*>(plan + off_pitems);
    a.scans = reinterpret_cast<const PScan*>(plan + off_pscan);
    a.hdr = reinterpret_cast<int*>(ws);
    a.flags = reinterpret_cast<uint64_t*>(ws + l.flags);
    a.aslots = reinterpret_cast<float*>(ws + l.aslots);
    a.pslots = reinterpret_cast<float*>(ws + l.pslots);
    a.final_state = final_state;
    a.ext_state = ext_state;
    a.out = static_cast<uint16_t*>(out);
    a.H = H;
    a.n_flags = info.piece_slots * H;
    a.n_slots = info.piece_slots;
    a.plan_hash = info.plan_hash;
    a.spin_limit = spin_limit;
    a.force_timeout = force_timeout ? 1 : 0;
    a.ordered = 1;
    const dim3 blk(kThreads);
    if (form == 1) {
        if (!(stages & LA_STAGE_ALL)) return LA_OK;
        a.n_work = info.piece_items * H;
        if (!ordered) {
            const int cap = resident_capacity();
            a.ordered = cap > 0 && a.n_work <= cap ? 0 : 1;
        }
        if (a.n_work > 0)
            hipLaunchKernelGGL(piece_kernel<kFused>, dim3(unsigned(a.n_work)), blk, 0, st, a.plan,
                           a.items, a.n_work, a.H, a.plan_hash, a.ordered, a);
        return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
    }
    if ((stages & LA_STAGE_STATES) && info.piece_block_items > 0) {
        a.n_work = info.piece_block_items * H;
        hipLaunchKernelGGL(piece_kernel<kStates>, dim3(unsigned(a.n_work)), blk, 0, st, a.plan,
                           a.items, a.n_work, a.H, a.plan_hash, a.ordered, a);
        if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    }
    if ((stages & LA_STAGE_PREFIX) && form == 3 && info.piece_scans > 0) {
        const la_status s = launch_prefix(plan + off_pscan, info.piece_scans, a.aslots,
                                          final_state, H, st, plan, a.hdr, info.plan_hash);
        if (s != LA_OK) return s;
    }
    if ((stages & LA_STAGE_OUTPUT) && info.piece_items > 0) {
        a.n_work = info.piece_items * H;
        if (form == 3)
            hipLaunchKernelGGL(piece_kernel<kOut3>, dim3(unsigned(a.n_work)), blk, 0, st, a.plan,
                           a.items, a.n_work, a.H, a.plan_hash, a.ordered, a);
        else
            hipLaunchKernelGGL(piece_kernel<kOut2>, dim3(unsigned(a.n_work)), blk, 0, st, a.plan,
                           a.items, a.n_work, a.H, a.plan_hash, a.ordered, a);
        if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    }
    return LA_OK;
}

}  // namespace piece
