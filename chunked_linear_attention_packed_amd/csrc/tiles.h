// Tile helpers shared by the gfx950 kernels of this library (scan.hip,
// attn.hip): vector types, MFMA and conversion wrappers, range-checked
// buffer windows over [T][H][D] tensors, and the staging of 64-token bf16
// tiles into LDS (row-major and transposed).  Internal header: every
// definition has internal linkage.
#ifndef LINATTN_TILES_H
#define LINATTN_TILES_H

#include <hip/hip_runtime.h>

#include <cstdint>

#include "linattn.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;   // 4 waves of 64
// s_waitcnt operand (gfx9 encoding): vector memory count 0, the export and
// LDS/scalar counts left at their maxima
constexpr int kWaitVmem0 = 0x0F70;
constexpr int kChunk = LA_CHUNK;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Two fp32 -> packed bf16 (low half = a), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_bf2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2_t));
}
__device__ __forceinline__ float bf_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Wave index as a wave-uniform (scalar) value, so that branches and buffer
// resources chosen by it stay scalar.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x)) >> 6;
}

// Workspace slot layout: element e of a d x d state is stored at
//   e = ((vb * NKB + kb) * 64 + lane) * 4 + j,   lane = 16 g + c
// holding S[kb*16 + 4g + j][vb*16 + c]: each lane keeps the 4 values of an
// accumulator tile in one 16-byte piece, and a tile is one coalesced
// 1 KB row of the slot.
template <int D>
__device__ __forceinline__ void slot_to_rc(int e, int& row, int& col) {
    constexpr int NKB = D / 16;
    const int j = e & 3;
    const int lane = (e >> 2) & 63;
    const int kb = (e >> 8) % NKB;
    const int vb = (e >> 8) / NKB;
    row = kb * 16 + 4 * (lane >> 4) + j;
    col = vb * 16 + (lane & 15);
}

// ---------------------------------------------------------------------------
// Range-checked chunk windows.  A chunk of `rows` tokens of a [T][H][D]
// tensor is addressed through a raw buffer resource whose size is
// rows*H*D*elem bytes from the chunk's first token: a token row r >= rows
// lies entirely past the end (its offset is at least rows*H*D*elem), so the
// hardware returns zeros for such loads and drops such stores.  Ragged last
// chunks need no branches.
// ---------------------------------------------------------------------------
// A window with rows <= 0 is empty: every load through it returns zeros
// without touching memory, so a prefetch past the last chunk can be issued
// unconditionally (no branch, hence no register merge that would force the
// compiler to wait for the loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, int64_t first_elem,
                                                             int elem_bytes, int rows, int H,
                                                             int D) {
    const char* p = static_cast<const char*>(base) + (rows > 0 ? first_elem * elem_bytes : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0,
                                             rows > 0 ? rows * H * D * elem_bytes : 0,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Stores of whole 128-byte output rows per instruction (buf_store16u, used
// by the row writers of the bf16 scan kernels) are nontemporal (cache policy
// nt): the outputs are written once and not read again by the pass, and
// streaming them past the L2 leaves no dirty output lines for the write-back
// at the end of the kernel (the 7,400-token pass: 24.1 -> 21.9 us).  Stores
// that write parts of lines (buf_store16, buf_store8) keep the default
// policy, so that the L2 merges a line's parts before it goes to memory: as
// nontemporal 8-byte stores, the attention kernel's output wrote 5.3 GB of
// HBM for 2.2 GB of output at the 272k-token pass.
constexpr int kAuxStream = 2;   // buffer-op cache policy: nt
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16u(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r, off, 0, kAuxStream);
}

__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 x) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, x), r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// bf16 tile staging.  A 64 x D tile is cut into R x 8 blocks (R tokens x 8
// features, R = 4 or 2); one lane loads a block as R row pieces of 16 bytes
// (8 lanes cover one D*2-byte row, so each load instruction reads whole cache
// lines) and writes it to LDS row-major and/or transposed.  The transpose is
// done in registers with v_perm_b32: column c of the block becomes R
// consecutive tokens, one R*2-byte LDS store.
// ---------------------------------------------------------------------------
// Row strides are padded so that the 16-byte fragment reads of the MFMA
// operands (lane 16g + c reads row c at column offset 16 g bytes) hit no LDS
// bank twice: measured on gfx950 with the bank-conflict counter, rows of 160
// bytes are conflict-free where rows of 144 bytes are not.  At d = 128 the
// workgroups of the output launch would no longer fit two per CU with the
// wider padding, so rows there keep 8 elements of padding.
template <int D, int R>
struct Stage {
    static constexpr int NCG = D / 8;           // 8-feature groups per row
    static constexpr int NB = (kChunk / R) * NCG;   // R x 8 blocks per 64-token tile
    static constexpr int PAD = D == 64 ? 16 : 8;
    static constexpr int LDR = D + PAD;         // row-major stride (elements)
    static constexpr int LDT = kChunk + PAD;    // transposed stride (elements)
    template <int W>
    static constexpr int LDV = W + PAD;         // row-major stride of a W-feature tile
};

// Column at which element k of row f of a row-major D-column state tile is
// kept: with 160-byte rows (d = 64), rows with bit 2 set swap 8-element
// halves of each 16-element group, which keeps the 8-byte stores of the
// state publication at the conflict level of the unswizzled 144-byte rows
// while the 16-byte reads stay conflict-free.  8-element groups stay
// contiguous, so a 16-byte read at an 8-aligned k reads k .. k + 7.
template <int D>
__device__ __forceinline__ int scol(int f, int k) {
    if constexpr (D == 64) return k ^ ((f & 4) << 1);
    return k;
}

template <int R>
struct BlkR {
    u32x4 r[R];  // r[i] = token i of the block, 8 bf16 features
};

template <int R>
__device__ __forceinline__ void load_blk(BlkR<R>& b, __amdgpu_buffer_rsrc_t rs, int rg, int cg,
                                         int H, int h, int D) {
#pragma unroll
    for (int i = 0; i < R; ++i)
        b.r[i] = buf_load16(rs, uint32_t((((rg * R + i) * H + h) * D + cg * 8) * 2));
}

template <int R>
__device__ __forceinline__ void store_rows(uint16_t* dst, const BlkR<R>& b, int rg, int cg,
                                           int ld) {
#pragma unroll
    for (int i = 0; i < R; ++i)
        *reinterpret_cast<u32x4*>(dst + (rg * R + i) * ld + cg * 8) = b.r[i];
}

// Transposed tiles [feature][token] (used by the split-precision kernels,
// whose fp32 data is split into bf16 terms while staging; the bf16 kernels
// read the same fragments from row-major tiles with tr_frag) hold the 64
// tokens of a row in the order
//   position(u) = 32 a + 8 c + 4 b + d   for   u = 32 a + 16 b + 4 c + d,
// so that the 8 tokens {32a + 16b + 4c + d : b, d} (two 4-token groups 16
// apart: the k-slots of lane group c in a K = 32 step whose two halves come
// from 16-row tiles 2a and 2a + 1) are 16 contiguous bytes.  Every consumer
// reads such 8-token groups: the carry K^T V (both operands in this order,
// so the contraction is unchanged) and the intra-chunk V^T P^T (whose P^T
// operand comes from accumulator tiles in exactly this slot order).  On top,
// the 16-position groups of a row are permuted by the feature's bits 4 and 5
// (the same for all 16 rows of a tile, so every reader addresses a tile with
// its first feature), which spreads the 8-byte column stores of one staging
// instruction over the LDS banks: measured, 3.8 instead of 11.3 conflict
// cycles per store against swapping 32-token halves by bit 4 alone.
__device__ __forceinline__ int tpos(int feature, int token) {
    const int pos = (token & 32) | ((token & 12) << 1) | ((token & 16) >> 2) | (token & 3);
    return pos ^ (feature & 48);
}

// dst[(cg*8 + c) * ld + tpos(cg*8 + c, rg*R) .. + R-1] = column c of the block
// (R = 2 or 4 consecutive tokens stay contiguous under tpos).
template <int R>
__device__ __forceinline__ void store_cols(uint16_t* dst, const BlkR<R>& b, int rg, int cg,
                                           int ld) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {   // features 2m (low halves) and 2m+1 (high halves)
        const int f0 = cg * 8 + 2 * m;   // f0 and f0 + 1 share bit 4
        const int t0 = tpos(f0, rg * R);
        if constexpr (R == 4) {
            const u32x2 ev{__builtin_amdgcn_perm(b.r[1][m], b.r[0][m], 0x05040100u),
                           __builtin_amdgcn_perm(b.r[3][m], b.r[2][m], 0x05040100u)};
            const u32x2 od{__builtin_amdgcn_perm(b.r[1][m], b.r[0][m], 0x07060302u),
                           __builtin_amdgcn_perm(b.r[3][m], b.r[2][m], 0x07060302u)};
            *reinterpret_cast<u32x2*>(dst + f0 * ld + t0) = ev;
            *reinterpret_cast<u32x2*>(dst + (f0 + 1) * ld + t0) = od;
        } else {
            static_assert(R == 2, "blocks of 2 or 4 tokens");
            *reinterpret_cast<uint32_t*>(dst + f0 * ld + t0) =
                __builtin_amdgcn_perm(b.r[1][m], b.r[0][m], 0x05040100u);
            *reinterpret_cast<uint32_t*>(dst + (f0 + 1) * ld + t0) =
                __builtin_amdgcn_perm(b.r[1][m], b.r[0][m], 0x07060302u);
        }
    }
}

__device__ __forceinline__ u32x4 cat2(u32x2 a, u32x2 b) { return u32x4{a[0], a[1], b[0], b[1]}; }

// ---------------------------------------------------------------------------
// Transposed fragments read from row-major [token][feature] tiles with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane
// group, lane 4a + e receives element e of the 8-byte pieces addressed by
// lanes a, a + 4, a + 8, a + 12 (probed on the GPU).  So if lane lam of the
// group addresses token t0 + lam / 4, features f0 + 4 (lam % 4) .. + 3, lane
// lam receives feature f0 + lam of tokens t0 .. t0 + 3.
// ---------------------------------------------------------------------------
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_tr4(const uint16_t* p) {
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
    return __builtin_bit_cast(u32x2, r);
}
// Operand fragment of a transposed 16-row tile (rows = features f0 .. f0+15,
// k = tokens) for K step ks of a 64-token chunk: lane 16 g + c gets row
// f0 + c, k-slots 4 h + j = token (2 ks + h) * 16 + 4 g + j (h = 0, 1,
// j = 0 .. 3) -- the slot order of the accumulator-layout P^T operand and the
// one the former transposed tiles stored.
__device__ __forceinline__ u32x4 tr_frag(const uint16_t* tile, int ld, int f0, int ks, int g,
                                         int c16) {
    const uint16_t* p = tile + (4 * g + (c16 >> 2)) * ld + f0 + 4 * (c16 & 3);
    return cat2(lds_tr4(p + (2 * ks) * 16 * ld), lds_tr4(p + (2 * ks + 1) * 16 * ld));
}

__device__ __forceinline__ u32x2 lds_u32x2(const uint16_t* p) {
    return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ u32x4 lds_u32x4(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// K and V blocks of one chunk: all D features of K, and the DVW features of V
// starting at feature vcg0 * 8 (a workgroup that computes only part of the
// output features needs only that part of V).  Block index b = tid + i*NT
// over [K | V]; each half is a whole number of waves, so the tile choice and
// whether a wave loads at all are wave-uniform.
template <int D, int DVW, int R, int NT>
struct KVStage {
    static constexpr int NCGK = D / 8, NCGV = DVW / 8;   // 8-feature groups per row
    static constexpr int NBK = (kChunk / R) * NCGK;     // K blocks
    static constexpr int NBV = (kChunk / R) * NCGV;     // V blocks
    static constexpr int NPER = (NBK + NBV + NT - 1) / NT;
    static_assert(NBK % 64 == 0 && NBV % 64 == 0, "K and V parts are whole waves");
};

template <int D, int DVW, int R, int NT, int NPER>
__device__ __forceinline__ void load_kv(BlkR<R> (&pre)[NPER], __amdgpu_buffer_rsrc_t rk,
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
        // selects, not branches: the loads stay unconditional
        const int rg = is_v ? wv / KS::NCGV : wk / KS::NCGK;
        const int cg = is_v ? vcg0 + wv % KS::NCGV : wk % KS::NCGK;
        load_blk<R>(pre[i], is_v ? rv : rk, rg, cg, H, h, D);
    }
}

// Registers -> LDS, both tiles row-major: K rows into sK (stride LDR), the
// workgroup's DVW features of V into sV (stride LDR of a DVW-wide tile);
// transposed operands are then read with tr_frag.
template <int D, int DVW, int R, int NT, int NPER,
          int LDVS = Stage<D, R>::template LDV<DVW>, int LDKS = Stage<D, R>::LDR>
__device__ __forceinline__ void stage_kv_rows(const BlkR<R> (&pre)[NPER], uint16_t* sK,
                                              uint16_t* sV) {
    using KS = KVStage<D, DVW, R, NT>;
    const int wbase = wave_id() * 64;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int b0 = wbase + i * NT;                      // wave-uniform
        if constexpr (NPER * NT > KS::NBK + KS::NBV)
            if (b0 >= KS::NBK + KS::NBV) break;
        if (b0 >= KS::NBK) {
            const int wv = b0 - KS::NBK + lane;
            store_rows<R>(sV, pre[i], wv / KS::NCGV, wv % KS::NCGV, LDVS);
        } else {
            const int wk = b0 + lane;
            store_rows<R>(sK, pre[i], wk / KS::NCGK, wk % KS::NCGK, LDKS);
        }
    }
}

}  // namespace

#endif  // LINATTN_TILES_H
