// Host-side packing and work planning for the packed linear-attention scan.
//
// Section "The Workload" of "Serving 0.88M TPS from Two RTXs and Mac Minis":
// a request is one long view plus short branches that attend to the view and
// never to each other.  Paragraph "Shared branch passes" (section "Kernels"):
// the branches of every request in a pass go through one packed forward.
// Section "Long Requests": a branch shard starts from the view's cached state.
//
// Everything here is integer bookkeeping on the host.  The output plan is the
// only metadata the device kernels read: one descriptor per work block, per
// delta block and per scanned segment.
#include <algorithm>
#include <array>
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "linattn.h"

namespace {

constexpr int32_t kPlanVersion = 5;

// Piece path (d = 64, bf16): blocks of LA_PIECE_BLOCK_CHUNKS chunks, each cut
// into pieces of LA_PIECE_CHUNKS chunks, one per wave of a 4-wave workgroup.
// Branches whose only block is a single piece are packed into workgroups of
// their own, four waves of them: two branches of at most one chunk share a
// wave, a branch of two chunks has one alone.
constexpr int32_t kPieceBlockTok = LA_PIECE_BLOCK_CHUNKS * LA_CHUNK;
constexpr int32_t kPieceTok = LA_PIECE_CHUNKS * LA_CHUNK;
constexpr int kPackWaves = 4;

// Waves of the packs, filled in branch order: a branch of at most one chunk
// joins the wave of the last such branch if that wave has room, else opens a
// new wave; a longer branch takes a new wave.
struct PackWaves {
    std::vector<std::array<int32_t, 2>> waves;
    int64_t open = -1;   // wave holding a lone branch of at most one chunk
    void add(int32_t block, int32_t len) {
        if (len <= LA_CHUNK && open >= 0) {
            waves[size_t(open)][1] = block;
            open = -1;
            return;
        }
        if (len <= LA_CHUNK) open = int64_t(waves.size());
        waves.push_back({block, -1});
    }
};

// FNV-1a over the plan words, with the hash word itself taken as zero.
uint32_t plan_hash(const int32_t* plan, int64_t words) {
    uint32_t h = 2166136261u;
    for (int64_t i = 0; i < words; ++i) {
        const uint32_t w = i == LA_PLAN_HASH_WORD ? 0u : uint32_t(plan[i]);
        for (int b = 0; b < 4; ++b) {
            h ^= (w >> (8 * b)) & 0xffu;
            h *= 16777619u;
        }
    }
    return h;
}

struct Seg {
    int32_t off, len, parent;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Validates a segment table and fills `info` and, when asked, the plan.
la_status plan_impl(int32_t n_seg, const int32_t* seg_offsets, const int32_t* branch_parent,
                    int32_t chunk, int32_t block_chunks, int32_t* view_ordinal, int32_t* plan,
                    la_pass_info* info) {
    if (!info) return LA_ERR_INVALID_ARG;
    if (chunk != LA_CHUNK) return LA_ERR_UNSUPPORTED;
    if (n_seg < 0 || block_chunks < 1 || block_chunks > (1 << 20)) return LA_ERR_INVALID_ARG;
    if (n_seg > 0 && (!seg_offsets || !branch_parent)) return LA_ERR_INVALID_ARG;
    if (n_seg == 0 && seg_offsets && seg_offsets[0] != 0) return LA_ERR_INVALID_ARG;

    const int64_t blk_tok = int64_t(block_chunks) * chunk;
    if (blk_tok > INT32_MAX) return LA_ERR_INVALID_ARG;

    std::vector<int32_t> ord(size_t(n_seg), -1);
    int32_t n_views = 0, n_branches = 0, n_ext = 0, max_len = 0;
    int64_t n_chunks = 0, n_view_chunks = 0;
    if (n_seg > 0 && seg_offsets[0] != 0) return LA_ERR_INVALID_ARG;
    for (int32_t s = 0; s < n_seg; ++s) {
        const int64_t len = int64_t(seg_offsets[s + 1]) - seg_offsets[s];
        if (len < 1) return LA_ERR_INVALID_ARG;
        if (len > max_len) max_len = int32_t(len);
        const int32_t p = branch_parent[s];
        if (p == -1) {
            ord[size_t(s)] = n_views++;
            n_view_chunks += ceil_div(len, chunk);
        } else {
            ++n_branches;
        }
        n_chunks += ceil_div(len, chunk);
    }
    // Parents are checked after all views are known: any order is accepted.
    for (int32_t s = 0; s < n_seg; ++s) {
        const int32_t p = branch_parent[s];
        if (p == -1) continue;
        if (p >= 0) {
            if (p >= n_seg || branch_parent[p] != -1) return LA_ERR_INVALID_ARG;
        } else {
            if (p < -2 - (INT32_MAX - 2)) return LA_ERR_INVALID_ARG;
            const int32_t e = -p - 2;
            if (e + 1 > n_ext) n_ext = e + 1;
        }
    }

    // Work blocks: views first (their blocks are the longest), then branches.
    // fused_reads counts the workspace slots the output launch reads per head
    // when it sums the block states itself (no prefix launch): block j of a
    // segment reads the j earlier slots of its segment, a branch of a view
    // also all slots of that view, and a view's last block its own slot.
    int64_t n_blocks = 0, n_delta = 0, n_scan = 0, fused_reads = 0;
    for (int pass = 0; pass < 2; ++pass) {
        for (int32_t s = 0; s < n_seg; ++s) {
            const int32_t p = branch_parent[s];
            const bool is_view = p == -1;
            if (is_view != (pass == 0)) continue;
            const int64_t len = int64_t(seg_offsets[s + 1]) - seg_offsets[s];
            const int64_t nb = ceil_div(len, blk_tok);
            n_blocks += nb;
            // A view needs every block's state (its total is final_state);
            // a branch needs all but its last block's.
            const int64_t nslots = is_view ? nb : nb - 1;
            n_delta += nslots;
            if (is_view || nslots >= 2) ++n_scan;
            fused_reads += nb * (nb - 1) / 2 + (is_view ? 1 : 0);
            if (p >= 0)
                fused_reads += nb * ceil_div(int64_t(seg_offsets[p + 1]) - seg_offsets[p], blk_tok);
        }
    }
    // Piece path tables: blocks of kPieceBlockTok tokens; a view's blocks all
    // get a state slot (its total is final_state, its branches start from
    // it), a branch's all but the last; branches whose only block is a
    // single piece are packed (PackWaves), everything else is one workgroup
    // per block.
    int64_t p_blocks = 0, p_slots = 0, p_scan = 0, p_block_items = 0;
    PackWaves pack_count;
    for (int32_t s = 0; s < n_seg; ++s) {
        const bool is_view = branch_parent[s] == -1;
        const int64_t len = int64_t(seg_offsets[s + 1]) - seg_offsets[s];
        const int64_t nb = ceil_div(len, kPieceBlockTok);
        const int64_t nslots = is_view ? nb : nb - 1;
        p_blocks += nb;
        p_slots += nslots;
        if (is_view || nslots >= 1) ++p_scan;
        if (!is_view && nb == 1 && len <= kPieceTok)
            pack_count.add(0, int32_t(len));
        else
            p_block_items += nb;
    }
    const int64_t p_items = p_block_items + ceil_div(int64_t(pack_count.waves.size()), kPackWaves);
    const int64_t words = int64_t(LA_PLAN_HEADER_WORDS) + n_blocks * LA_PLAN_BLOCK_WORDS +
                          n_delta * LA_PLAN_DELTA_WORDS + n_scan * LA_PLAN_SCAN_WORDS +
                          p_blocks * LA_PLAN_BLOCK_WORDS + p_items * LA_PLAN_ITEM_WORDS +
                          p_scan * LA_PLAN_SCAN_WORDS;
    if (words > INT32_MAX || n_chunks > INT32_MAX) return LA_ERR_INVALID_ARG;

    la_pass_info inf;
    std::memset(&inf, 0, sizeof(inf));
    inf.n_requests = 0;
    inf.n_segments = n_seg;
    inf.n_views = n_views;
    inf.n_branches = n_branches;
    inf.n_ext = n_ext;
    inf.n_tokens = n_seg > 0 ? seg_offsets[n_seg] : 0;
    inf.chunk = chunk;
    inf.block_chunks = block_chunks;
    inf.n_chunks = int32_t(n_chunks);
    inf.n_view_chunks = int32_t(n_view_chunks);
    inf.n_blocks = int32_t(n_blocks);
    inf.n_delta = int32_t(n_delta);
    inf.n_scan = int32_t(n_scan);
    inf.plan_words = int32_t(words);
    inf.max_seg_tokens = max_len;
    inf.fused_slot_reads = int32_t(std::min<int64_t>(fused_reads, INT32_MAX));
    inf.piece_blocks = int32_t(p_blocks);
    inf.piece_items = int32_t(p_items);
    inf.piece_block_items = int32_t(p_block_items);
    inf.piece_slots = int32_t(p_slots);
    inf.piece_scans = int32_t(p_scan);

    if (view_ordinal)
        for (int32_t s = 0; s < n_seg; ++s) view_ordinal[s] = ord[size_t(s)];

    if (plan) {
        const int32_t off_blocks = LA_PLAN_HEADER_WORDS;
        const int32_t off_delta = off_blocks + int32_t(n_blocks) * LA_PLAN_BLOCK_WORDS;
        const int32_t off_scan = off_delta + int32_t(n_delta) * LA_PLAN_DELTA_WORDS;
        const int32_t off_pblocks = off_scan + int32_t(n_scan) * LA_PLAN_SCAN_WORDS;
        const int32_t off_pitems = off_pblocks + int32_t(p_blocks) * LA_PLAN_BLOCK_WORDS;
        const int32_t off_pscan = off_pitems + int32_t(p_items) * LA_PLAN_ITEM_WORDS;
        int32_t* h = plan;
        std::memset(h, 0, sizeof(int32_t) * LA_PLAN_HEADER_WORDS);
        h[0] = LA_PLAN_MAGIC;
        h[1] = kPlanVersion;
        h[2] = int32_t(n_blocks);
        h[3] = int32_t(n_delta);
        h[4] = int32_t(n_scan);
        h[5] = chunk;
        h[6] = block_chunks;
        h[7] = inf.n_tokens;
        h[8] = off_blocks;
        h[9] = off_delta;
        h[10] = off_scan;
        h[11] = n_ext;
        h[12] = n_views;
        h[13] = inf.fused_slot_reads;
        h[15] = int32_t(p_blocks);
        h[16] = int32_t(p_items);
        h[17] = int32_t(p_block_items);
        h[18] = int32_t(p_slots);
        h[19] = int32_t(p_scan);
        h[20] = off_pblocks;
        h[21] = off_pitems;
        h[22] = off_pscan;
        int32_t* blk = plan + off_blocks;
        int32_t* del = plan + off_delta;
        int32_t* scn = plan + off_scan;
        int32_t slot = 0;
        for (int pass = 0; pass < 2; ++pass) {
            for (int32_t s = 0; s < n_seg; ++s) {
                const int32_t p = branch_parent[s];
                const bool is_view = p == -1;
                if (is_view != (pass == 0)) continue;
                const int32_t off = seg_offsets[s];
                const int32_t len = seg_offsets[s + 1] - off;
                const int32_t nb = int32_t(ceil_div(len, blk_tok));
                const int32_t nslots = is_view ? nb : nb - 1;
                const int32_t seed = is_view ? -1 : (p >= 0 ? ord[size_t(p)] : p);
                const int32_t slot0 = nslots > 0 ? slot : -1;
                for (int32_t j = 0; j < nb; ++j) {
                    const int32_t tok0 = off + int32_t(j * blk_tok);
                    const int32_t ntok = int32_t(len - j * blk_tok < blk_tok ? len - j * blk_tok
                                                                             : blk_tok);
                    blk[0] = tok0;
                    blk[1] = ntok;
                    blk[2] = j >= 1 ? slot + j - 1 : -1;
                    blk[3] = j < nslots ? slot + j : -1;
                    blk[4] = seed;
                    blk[5] = s;
                    blk[6] = slot0;
                    blk[7] = is_view && j == nb - 1 ? ord[size_t(s)] : -1;
                    blk += LA_PLAN_BLOCK_WORDS;
                    if (j < nslots) {
                        del[0] = tok0;
                        del[1] = ntok;
                        del[2] = slot + j;
                        del[3] = s;
                        del += LA_PLAN_DELTA_WORDS;
                    }
                }
                if (is_view || nslots >= 2) {
                    scn[0] = slot;
                    scn[1] = nslots;
                    scn[2] = is_view ? ord[size_t(s)] : -1;
                    scn[3] = s;
                    scn += LA_PLAN_SCAN_WORDS;
                }
                slot += nslots;
            }
        }
        // Piece path.  Blocks: views (segment order), then branches; each
        // block {tok0, ntok, slot, seed, seg, slot0, j, final_row}.  Scans:
        // the views in ordinal order first (a branch finds its view's slots
        // at pscan[seed]), then branches with slots.  Items: one per
        // non-packed block in block order, then the packs.
        int32_t* pb = plan + off_pblocks;
        int32_t* pit = plan + off_pitems;
        int32_t* psc = plan + off_pscan;
        PackWaves packs;
        int32_t pslot = 0, pblock = 0;
        std::vector<int32_t> view_scan(size_t(n_views > 0 ? n_views : 0), -1);
        for (int pass = 0; pass < 2; ++pass) {
            for (int32_t s = 0; s < n_seg; ++s) {
                const int32_t p = branch_parent[s];
                const bool is_view = p == -1;
                if (is_view != (pass == 0)) continue;
                const int32_t off = seg_offsets[s];
                const int32_t len = seg_offsets[s + 1] - off;
                const int32_t nb = int32_t(ceil_div(len, kPieceBlockTok));
                const int32_t nslots = is_view ? nb : nb - 1;
                const int32_t seed = is_view ? -1 : (p >= 0 ? ord[size_t(p)] : p);
                const int32_t slot0 = nslots > 0 ? pslot : -1;
                const bool pack = !is_view && nb == 1 && len <= kPieceTok;
                for (int32_t j = 0; j < nb; ++j) {
                    const int32_t tok0 = off + j * kPieceBlockTok;
                    const int32_t ntok = std::min(kPieceBlockTok, len - j * kPieceBlockTok);
                    pb[0] = tok0;
                    pb[1] = ntok;
                    pb[2] = j < nslots ? pslot + j : -1;
                    pb[3] = seed;
                    pb[4] = s;
                    pb[5] = slot0;
                    pb[6] = j;
                    pb[7] = is_view && j == nb - 1 ? ord[size_t(s)] : -1;
                    pb += LA_PLAN_BLOCK_WORDS;
                    if (pack) {
                        packs.add(pblock, len);
                    } else {
                        // a block item carries a copy of its block, so a
                        // workgroup reads one record before its first load
                        int32_t* it = pit;
                        it[0] = LA_ITEM_BLOCK;
                        it[1] = 1;
                        it[2] = pblock;
                        it[3] = -1;
                        std::memcpy(it + 4, pb - LA_PLAN_BLOCK_WORDS,
                                    sizeof(int32_t) * LA_PLAN_BLOCK_WORDS);
                        pit += LA_PLAN_ITEM_WORDS;
                    }
                    ++pblock;
                }
                if (is_view || nslots >= 1) {
                    psc[0] = pslot;
                    psc[1] = nslots;
                    psc[2] = is_view ? ord[size_t(s)] : -1;
                    psc[3] = s;
                    psc += LA_PLAN_SCAN_WORDS;
                }
                pslot += nslots;
            }
        }
        const size_t nw = packs.waves.size();
        for (size_t i = 0; i < nw; i += kPackWaves) {
            int32_t* it = pit;
            std::memset(it, 0, sizeof(int32_t) * LA_PLAN_ITEM_WORDS);
            it[0] = LA_ITEM_PACK;
            it[1] = int32_t(std::min<size_t>(kPackWaves, nw - i));
            for (int w = 0; w < kPackWaves; ++w)
                for (int b = 0; b < 2; ++b)
                    it[2 + 2 * w + b] = i + size_t(w) < nw ? packs.waves[i + size_t(w)][size_t(b)] : -1;
            pit += LA_PLAN_ITEM_WORDS;
        }
        const uint32_t hash = plan_hash(plan, words);
        h[LA_PLAN_HASH_WORD] = int32_t(hash);
        inf.plan_hash = int32_t(hash);
    }
    inf.info_check = int32_t(la_info_checksum(&inf));
    *info = inf;
    return LA_OK;
}

}  // namespace

// Checksum of an la_pass_info's fields (all but info_check itself): a copy
// that was edited by hand, or fields mixed from two passes, do not match.
extern "C" uint32_t la_info_checksum(const la_pass_info* info) {
    la_pass_info c = *info;
    c.info_check = 0;
    const unsigned char* b = reinterpret_cast<const unsigned char*>(&c);
    uint32_t h = 2166136261u ^ 0x9e3779b9u;
    for (size_t i = 0; i < sizeof(c); ++i) {
        h ^= b[i];
        h *= 16777619u;
    }
    return h;
}

// Work-block size (chunks per block) for a pass of H heads: the largest
// power of two up to kGroupMaxG whose blocks times H reach kGroupTarget
// workgroups (about one per compute unit of an MI355X), 1 if none; then,
// while the views alone still give kLongTarget workgroups at twice the size
// (8 per compute unit, so the pass is far from bound by its longest chain),
// doubled up to kLongMaxG.  Larger blocks carry the state in registers
// longer (fewer block states to write, scan and read, fewer prologues);
// smaller ones give more workgroups and shorter serial chains.  Measured on
// MI355X: the 7,400-token pass is fastest at 8, a view of 18,000 tokens with
// 256 branches at 16 (144 view workgroups at 32: 93.7 -> 102.6 us), the
// 272k-token pass of 32 requests (H 32, d 128) at 64 (3408 / 3276 / 3225 us
// at 16 / 32 / 64).
extern "C" la_status la_choose_block_chunks(int32_t n_segments, const int32_t* seg_offsets,
                                            const int32_t* branch_parent, int32_t heads,
                                            int32_t* block_chunks) {
    constexpr int64_t kGroupTarget = 300, kLongTarget = 2048;
    constexpr int32_t kGroupMaxG = 16, kLongMaxG = 64;
    if (!block_chunks || heads < 1 || n_segments < 0) return LA_ERR_INVALID_ARG;
    if (n_segments > 0 && (!seg_offsets || !branch_parent)) return LA_ERR_INVALID_ARG;
    std::vector<int64_t> chunks(static_cast<size_t>(n_segments));
    for (int32_t s = 0; s < n_segments; ++s) {
        const int64_t len = int64_t(seg_offsets[s + 1]) - seg_offsets[s];
        if (len < 1) return LA_ERR_INVALID_ARG;
        chunks[size_t(s)] = ceil_div(len, LA_CHUNK);
    }
    auto blocks = [&](int32_t g, bool views_only) {
        int64_t nb = 0;
        for (int32_t s = 0; s < n_segments; ++s)
            if (!views_only || branch_parent[s] == -1) nb += ceil_div(chunks[size_t(s)], g);
        return nb;
    };
    int32_t g = kGroupMaxG;
    while (g > 1 && blocks(g, false) * heads < kGroupTarget) g /= 2;
    if (g == kGroupMaxG)
        while (2 * g <= kLongMaxG && blocks(2 * g, true) * heads >= kLongTarget) g *= 2;
    *block_chunks = g;
    return LA_OK;
}

extern "C" la_status la_plan_segments(int32_t n_segments, const int32_t* seg_offsets,
                                      const int32_t* branch_parent, int32_t chunk,
                                      int32_t block_chunks, int32_t* view_ordinal,
                                      int32_t* plan, la_pass_info* info) {
    return plan_impl(n_segments, seg_offsets, branch_parent, chunk, block_chunks, view_ordinal,
                     plan, info);
}

extern "C" la_status la_pack_pass_ext(int32_t n_requests, const int32_t* view_len,
                                      const int32_t* branch_count, const int32_t* branch_len,
                                      const int32_t* ext_row, int32_t chunk,
                                      int32_t block_chunks, int32_t* seg_offsets,
                                      int32_t* branch_parent, int32_t* view_ordinal,
                                      int32_t* plan, la_pass_info* info) {
    if (!info || n_requests < 0) return LA_ERR_INVALID_ARG;
    if (n_requests > 0 && (!view_len || !branch_count)) return LA_ERR_INVALID_ARG;
    if (chunk != LA_CHUNK) return LA_ERR_UNSUPPORTED;
    int64_t n_br = 0;
    for (int32_t r = 0; r < n_requests; ++r) {
        if (view_len[r] < 0 || branch_count[r] < 0) return LA_ERR_INVALID_ARG;
        if (view_len[r] == 0 && branch_count[r] == 0) return LA_ERR_INVALID_ARG;
        if (view_len[r] == 0 && ext_row && (ext_row[r] < 0 || ext_row[r] > (1 << 30)))
            return LA_ERR_INVALID_ARG;
        n_br += branch_count[r];
    }
    if (n_br > 0 && !branch_len) return LA_ERR_INVALID_ARG;
    if (n_br > INT32_MAX / 2) return LA_ERR_INVALID_ARG;

    // Build the segment table: request by request, view then branches.
    std::vector<int32_t> off;
    std::vector<int32_t> par;
    off.reserve(size_t(n_requests + n_br + 1));
    par.reserve(size_t(n_requests + n_br));
    off.push_back(0);
    int64_t tok = 0;
    int32_t n_ext = 0;
    int64_t b = 0;
    for (int32_t r = 0; r < n_requests; ++r) {
        int32_t seed;
        if (view_len[r] > 0) {
            seed = int32_t(par.size());
            par.push_back(-1);
            tok += view_len[r];
            if (tok > INT32_MAX) return LA_ERR_INVALID_ARG;
            off.push_back(int32_t(tok));
        } else {
            // a shard request: its branches start from ext_state row
            // ext_row[r], or from the next row in order
            seed = -2 - (ext_row ? ext_row[r] : n_ext);
            ++n_ext;
        }
        for (int32_t i = 0; i < branch_count[r]; ++i, ++b) {
            if (branch_len[b] < 1) return LA_ERR_INVALID_ARG;
            par.push_back(seed);
            tok += branch_len[b];
            if (tok > INT32_MAX) return LA_ERR_INVALID_ARG;
            off.push_back(int32_t(tok));
        }
    }
    const int32_t n_seg = int32_t(par.size());
    la_pass_info inf;
    la_status st = plan_impl(n_seg, off.data(), par.data(), chunk, block_chunks, view_ordinal,
                             plan, &inf);
    if (st != LA_OK) return st;
    inf.n_requests = n_requests;
    inf.info_check = int32_t(la_info_checksum(&inf));
    if (seg_offsets) std::memcpy(seg_offsets, off.data(), sizeof(int32_t) * off.size());
    if (branch_parent && n_seg > 0) std::memcpy(branch_parent, par.data(), sizeof(int32_t) * par.size());
    *info = inf;
    return LA_OK;
}

extern "C" la_status la_pack_pass(int32_t n_requests, const int32_t* view_len,
                                  const int32_t* branch_count, const int32_t* branch_len,
                                  int32_t chunk, int32_t block_chunks, int32_t* seg_offsets,
                                  int32_t* branch_parent, int32_t* view_ordinal, int32_t* plan,
                                  la_pass_info* info) {
    return la_pack_pass_ext(n_requests, view_len, branch_count, branch_len, nullptr, chunk,
                            block_chunks, seg_offsets, branch_parent, view_ordinal, plan, info);
}

extern "C" la_status la_attn_plan_ext(int32_t n_segments, const int32_t* seg_offsets,
                                      const int32_t* branch_parent, int32_t n_ext,
                                      const int32_t* ext_len, const int32_t* ext_start,
                                      int32_t ext_tokens, int32_t* items, int32_t* n_items) {
    if (!n_items || n_segments < 0 || n_ext < 0 || ext_tokens < 0) return LA_ERR_INVALID_ARG;
    if (n_segments > 0 && (!seg_offsets || !branch_parent)) return LA_ERR_INVALID_ARG;
    if (n_ext > 0 && !ext_len) return LA_ERR_INVALID_ARG;
    if (n_segments > 0 && seg_offsets[0] != 0) return LA_ERR_INVALID_ARG;
    for (int32_t s = 0; s < n_segments; ++s)
        if (seg_offsets[s + 1] <= seg_offsets[s]) return LA_ERR_INVALID_ARG;
    // external view e is tokens [ext_off[e], ext_off[e] + ext_len[e]) of ext_k / ext_v:
    // at ext_start[e], or concatenated in order when ext_start is NULL; every
    // view lies inside the ext_tokens rows the arrays hold
    std::vector<int64_t> ext_off(size_t(n_ext) + 1, 0);
    for (int32_t e = 0; e < n_ext; ++e) {
        if (ext_len[e] < 1) return LA_ERR_INVALID_ARG;
        if (ext_start) {
            if (ext_start[e] < 0) return LA_ERR_INVALID_ARG;
            ext_off[e] = ext_start[e];
        }
        if (ext_off[e] + ext_len[e] > ext_tokens) return LA_ERR_INVALID_ARG;
        if (!ext_start) ext_off[e + 1] = ext_off[e] + ext_len[e];
    }
    struct Item {
        int32_t w[8];
        int64_t keys;
        int64_t group;   // the segment whose keys the item reads first (its view, or itself)
        int64_t gkeys;   // the longest key range of the group
    };
    std::vector<Item> out;
    for (int32_t s = 0; s < n_segments; ++s) {
        const int32_t p = branch_parent[s];
        int32_t view0 = 0, view_len = 0, src = LA_ATTN_NO_VIEW;
        if (p >= 0) {
            if (p >= n_segments || branch_parent[p] != -1) return LA_ERR_INVALID_ARG;
            view0 = seg_offsets[p];
            view_len = seg_offsets[p + 1] - seg_offsets[p];
            src = LA_ATTN_PACKED_VIEW;
        } else if (p <= -2) {
            const int64_t e = -int64_t(p) - 2;
            if (e >= n_ext) return LA_ERR_INVALID_ARG;
            view0 = int32_t(ext_off[size_t(e)]);
            view_len = ext_len[e];
            src = LA_ATTN_EXT_VIEW;
        }
        const int32_t a = seg_offsets[s], b = seg_offsets[s + 1];
        for (int32_t q0 = a; q0 < b; q0 += LA_CHUNK) {
            const int32_t nq = std::min(LA_CHUNK, b - q0);
            Item it{{q0, nq, a, view0, view_len, src, 0, 0}, int64_t(view_len) + (q0 + nq - a),
                    p >= 0 ? int64_t(p) : p <= -2 ? int64_t(n_segments) - p : int64_t(s), 0};
            out.push_back(it);
        }
    }
    // Items that read the same view's keys (the view's own query blocks and
    // its branches') are consecutive: workgroups dispatched together then
    // stream the same key blocks and share them in the L2, which a view's
    // keys at d = 128 (up to 8 MB per head) do not fit otherwise.  Groups
    // with the longest key range go first, and within a group the longest
    // items, so the long items start before the short ones.
    {
        std::unordered_map<int64_t, int64_t> gk;
        for (const Item& x : out) gk[x.group] = std::max(gk[x.group], x.keys);
        for (Item& x : out) x.gkeys = gk[x.group];
    }
    std::stable_sort(out.begin(), out.end(), [](const Item& x, const Item& y) {
        if (x.gkeys != y.gkeys) return x.gkeys > y.gkeys;
        if (x.group != y.group) return x.group < y.group;
        return x.keys > y.keys;
    });
    if (out.size() > size_t(INT32_MAX / LA_ATTN_ITEM_WORDS)) return LA_ERR_INVALID_ARG;
    if (items)
        for (size_t i = 0; i < out.size(); ++i)
            std::memcpy(items + i * LA_ATTN_ITEM_WORDS, out[i].w, sizeof(out[i].w));
    *n_items = int32_t(out.size());
    return LA_OK;
}

extern "C" la_status la_attn_plan(int32_t n_segments, const int32_t* seg_offsets,
                                  const int32_t* branch_parent, int32_t n_ext,
                                  const int32_t* ext_len, int32_t* items, int32_t* n_items) {
    if (n_ext < 0 || (n_ext > 0 && !ext_len)) return LA_ERR_INVALID_ARG;
    int64_t total = 0;
    for (int32_t e = 0; e < n_ext; ++e) {
        if (ext_len[e] < 1) return LA_ERR_INVALID_ARG;
        total += ext_len[e];
        if (total > INT32_MAX) return LA_ERR_INVALID_ARG;
    }
    return la_attn_plan_ext(n_segments, seg_offsets, branch_parent, n_ext, ext_len, nullptr,
                            int32_t(total), items, n_items);
}

extern "C" const char* la_status_string(la_status status) {
    switch (status) {
        case LA_OK: return "ok";
        case LA_ERR_INVALID_ARG: return "invalid argument";
        case LA_ERR_UNSUPPORTED: return "unsupported dtype, head dim or chunk size";
        case LA_ERR_WORKSPACE: return "workspace missing or too small";
        case LA_ERR_HIP: return "HIP runtime error";
        case LA_ERR_PLAN:
            return "the device plan does not belong to this pass info (rebuild it with the planner)";
        case LA_ERR_TIMEOUT:
            return "a wait inside the single-launch scan gave up (its outputs are not valid)";
        case LA_ERR_TOO_LARGE:
            return "the pass needs more workspace than the library's built-in scratch array holds";
        default: return "unknown status";
    }
}
