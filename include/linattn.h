/*
 * linattn.h -- C ABI of the packed chunked causal linear-attention scan
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  The page "Serving 0.88M TPS from Two RTXs and
 * Mac Minis" describes a scoring pass in which each request is one long view
 * followed by many short branches; branches attend to their own view but never
 * to each other (section "The Workload").  Most layers are linear attention,
 * evaluated in 64-token chunks with a few 64x64 matrix products each, and one
 * scan covers every view of a pass in three launches (section "Kernels",
 * paragraphs "Tensor cores for linear attention" and "One scan per pass").
 * The branches of all requests share one packed forward (paragraph "Shared
 * branch passes").  A branch shard can start from the view's cached
 * linear-attention state instead of the view's tokens (section "Long
 * Requests").  The page writes no equation; this library computes, per head,
 * the plain unnormalised causal form
 *
 *     S_t = S_{t-1} + k_t^T v_t,      o_t = q_t S_t        (fp32 state)
 *
 * with S = 0 at the start of each view and S = the final state of the parent
 * view (or a caller-supplied state) at the start of each branch.
 *
 * Conventions common to every call
 *   - All integers are int32 unless stated.  Tokens are packed segment after
 *     segment; q, k, v and out are dense, token-major [T][H][d] arrays.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are HIP device
 *     memory of the current device.  The caller owns every buffer; the library
 *     allocates nothing and keeps no state between calls, except the built-in
 *     scratch array behind la_scan_packed_noalloc (for callers that cannot
 *     allocate).
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).
 *     Device calls only enqueue work and return; results are ready when the
 *     stream is synchronised.  Calls on different streams may overlap.
 *   - Every call returns an la_status.  Argument, shape and dtype errors are
 *     found on the host before anything is enqueued and leave every output
 *     untouched.  Device-side metadata (the plan) is trusted: build it with
 *     la_pack_pass or la_plan_segments.  A failed launch returns LA_ERR_HIP;
 *     an asynchronous device fault surfaces at the caller's next
 *     synchronisation.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t la_status;
enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARG = 1,   /* NULL pointer, bad length, bad parent, ... */
    LA_ERR_UNSUPPORTED = 2,   /* dtype, head dim or chunk size not built   */
    LA_ERR_WORKSPACE = 3,     /* workspace missing or too small            */
    LA_ERR_HIP = 4,           /* a HIP runtime call or launch failed       */
    LA_ERR_TOO_LARGE = 5,     /* the pass needs more scratch memory than the
                                 library's built-in array holds
                                 (la_scan_packed_noalloc)                  */
    LA_ERR_PLAN = 6,          /* the device plan does not belong to the
                                 la_pass_info given with it (reported by
                                 the kernels, see la_scan_status)          */
    LA_ERR_TIMEOUT = 7        /* a bounded wait of the single-launch scan
                                 gave up (see la_scan_status)              */
};

typedef int32_t la_dtype;
enum {
    LA_F32 = 0,               /* fp32 q/k/v/out, fp32 MFMA products        */
    LA_BF16 = 1,              /* bf16 q/k/v/out, fp32 state and accumulate */
    LA_F32_SPLIT = 2          /* fp32 q/k/v/out; every product as three bf16
                                 MFMAs over hi/lo splits of its operands
                                 (hi.hi + hi.lo + lo.hi), the analogue of the
                                 page's split 3xtf32 (section "Kernels",
                                 paragraph "Tensor cores for linear
                                 attention"); fp32 state and accumulate   */
};

/* Chunk size of the scan (tokens per chunk tile).  Section "Kernels" of the
 * page evaluates linear attention in 64-token chunks; only 64 is built. */
#define LA_CHUNK 64

/* Magic word at plan[0]; plan[LA_PLAN_HASH_WORD] holds a hash of the whole
 * plan (taken with that word as zero), also kept in la_pass_info.plan_hash. */
#define LA_PLAN_MAGIC 0x4C41504E
#define LA_PLAN_HASH_WORD 14
#define LA_PLAN_HEADER_WORDS 32
#define LA_PLAN_BLOCK_WORDS 8
#define LA_PLAN_DELTA_WORDS 4
#define LA_PLAN_SCAN_WORDS 4
#define LA_PLAN_ITEM_WORDS 12
#define LA_ITEM_BLOCK 0
#define LA_ITEM_PACK 1
/* The piece path (d = 64, bf16 inputs) cuts every segment into blocks of
 * LA_PIECE_BLOCK_CHUNKS chunks and every block into pieces of
 * LA_PIECE_CHUNKS chunks, one piece per wave of a 4-wave workgroup. */
#define LA_PIECE_CHUNKS 2
#define LA_PIECE_BLOCK_CHUNKS 8

/* Shape summary of one packed pass, filled by la_pack_pass or
 * la_plan_segments and read by la_scan_workspace_size and la_scan_packed. */
typedef struct {
    int32_t n_requests;       /* requests given to la_pack_pass (0 for la_plan_segments) */
    int32_t n_segments;       /* views + branches                              */
    int32_t n_views;          /* rows of final_state                           */
    int32_t n_branches;
    int32_t n_ext;            /* rows of ext_state the pass reads              */
    int32_t n_tokens;         /* T                                             */
    int32_t chunk;            /* C, tokens per chunk (LA_CHUNK)                */
    int32_t block_chunks;     /* G, chunks per work block                      */
    int32_t n_chunks;         /* sum over segments of ceil(len / C)            */
    int32_t n_view_chunks;    /* the same over views only                      */
    int32_t n_blocks;         /* work blocks (launch 3 runs blocks x H groups) */
    int32_t n_delta;          /* blocks whose state launch 1 computes          */
    int32_t n_scan;           /* segments launch 2 scans                       */
    int32_t plan_words;       /* int32 words of the plan                       */
    int32_t max_seg_tokens;   /* longest segment                               */
    int32_t fused_slot_reads; /* workspace slots read per head by the output
                                 launch when it sums the block states itself
                                 (two-launch form, see la_scan_packed),
                                 saturated at INT32_MAX                        */
    int32_t piece_blocks;     /* piece path: blocks of LA_PIECE_BLOCK_CHUNKS    */
    int32_t piece_items;      /* piece path: workgroup items (x H heads)        */
    int32_t piece_block_items;/* piece path: items holding one block (the
                                 others hold up to four one-piece branches)    */
    int32_t piece_slots;      /* piece path: block states kept per head        */
    int32_t piece_scans;      /* piece path: segments with block states        */
    int32_t plan_hash;        /* hash of the plan the planner wrote            */
    int32_t info_check;       /* la_info_checksum of the other fields          */
    int32_t reserved[1];
} la_pass_info;

/* Checksum of an la_pass_info, over every field but info_check.  The planners
 * store it in info_check; la_scan_packed rejects an info whose fields no
 * longer match it (edited, or mixed from two passes).  Host only. */
uint32_t la_info_checksum(const la_pass_info* info);

/*
 * la_plan_segments -- build the device work plan of a pass from its segment
 * table (any segment order whose parents are views).
 *
 *   n_segments       number of segments (>= 0)
 *   seg_offsets      host [n_segments + 1]: token offset of each segment;
 *                    seg_offsets[0] == 0, strictly increasing (every segment
 *                    holds >= 1 token), total < 2^31
 *   branch_parent    host [n_segments]: -1 for a view; for a branch either the
 *                    segment index of its view (a segment whose parent is -1)
 *                    or -2 - e to start from row e of ext_state (shard pass,
 *                    section "Long Requests")
 *   chunk            tokens per chunk; must be LA_CHUNK
 *   block_chunks     G >= 1: chunks per work block.  A block is scanned by one
 *                    workgroup per head carrying the state in registers;
 *                    larger G means less state traffic, fewer workgroups
 *   view_ordinal     host [n_segments] or NULL: row of final_state of a view,
 *                    -1 for a branch
 *   plan             host [info->plan_words] or NULL: the plan to upload to
 *                    the device as int32 (layout below)
 *   info             host, required: filled on success
 * Call with view_ordinal = plan = NULL to learn info->plan_words first, then
 * again with the same table and block_chunks and buffers of that size (the
 * library cannot see their capacity).
 * Errors: LA_ERR_INVALID_ARG (bad table), LA_ERR_UNSUPPORTED (chunk).
 *
 * Plan layout (int32 words):
 *   [0..31]   header: magic, version 5, n_blocks, n_delta, n_scan, chunk,
 *             block_chunks, n_tokens, off_blocks, off_delta, off_scan, n_ext,
 *             n_views, fused_slot_reads, plan hash, then for the piece path
 *             piece_blocks, piece_items, piece_block_items, piece_slots,
 *             piece_scans, off_pblocks, off_pitems, off_pscan, 0 ...
 *   blocks    n_blocks x 8:
 *             {tok0, ntok, sin_slot, delta_slot, seed, seg, slot0, final_row}
 *             sin_slot   workspace slot holding the segment-local state before
 *                        the block (after the prefix launch), -1 for a
 *                        segment's first block
 *             delta_slot slot that launch 1 fills with the block's own
 *                        sum of k_t^T v_t, -1 if no later block needs it
 *             seed       -1: start from zero (view); v >= 0: start from
 *                        final_state row v; <= -2: ext_state row -seed-2
 *             slot0      first slot of the block's segment (-1: none); in the
 *                        two-launch form the block sums slots slot0 ..
 *                        sin_slot itself
 *             final_row  final_state row that a view's last block writes in
 *                        the two-launch form; -1 for every other block
 *   delta     n_delta x 4: {tok0, ntok, slot, seg}
 *   scan      n_scan x 4:  {first_slot, n_slots, final_row (-1: branch), seg};
 *             the first n_views entries are the views, in ordinal order (the
 *             two-launch form finds a branch's view slots at scan[seed])
 *   pblocks   piece_blocks x 8: {tok0, ntok, slot, seed, seg, slot0, j,
 *             final_row} -- blocks of LA_PIECE_BLOCK_CHUNKS chunks; slot: the
 *             block's state slot (-1: none needed), slot0: the segment's first
 *             slot, j: the block's position in its segment
 *   pitems    piece_items x 12 -- kind LA_ITEM_BLOCK: {kind, 1, b0, -1,
 *             pblocks[b0]} (one block, its 8 words copied into the item;
 *             wave w takes its piece w); kind LA_ITEM_PACK: {kind, n, b0, ..,
 *             b7, 0, 0}, branches whose only block is one piece,
 *             n waves of them: wave w takes block b_2w and, when b_2w+1 is
 *             not -1, block b_2w+1 after it (two branches of at most one
 *             chunk each share a wave; a branch of two chunks has one alone).
 *             Block items first, in block order, then the packs.
 *   pscan     piece_scans x 4, as scan, for the piece path's slots
 * View blocks come first (longest work first), then branch blocks.
 */
la_status la_plan_segments(int32_t n_segments, const int32_t* seg_offsets,
                           const int32_t* branch_parent, int32_t chunk,
                           int32_t block_chunks, int32_t* view_ordinal,
                           int32_t* plan, la_pass_info* info);

/*
 * la_choose_block_chunks -- a work-block size (chunks per block, the
 * block_chunks argument of the planners) for a pass of `heads` heads: the
 * largest power of two up to 16 whose blocks times heads reach 300
 * workgroups (1 if none), doubled up to 64 while the view blocks alone
 * still give 2048 workgroups.  Host only.
 *   n_segments, seg_offsets, branch_parent   the segment table, as for
 *                                            la_plan_segments
 *   heads                                    H >= 1
 *   block_chunks                             host, out
 * Errors: LA_ERR_INVALID_ARG (NULL, heads < 1, an empty segment).
 */
la_status la_choose_block_chunks(int32_t n_segments, const int32_t* seg_offsets,
                                 const int32_t* branch_parent, int32_t heads,
                                 int32_t* block_chunks);

/*
 * la_pack_pass -- pack request shapes into segments and build the plan
 * (section "The Workload": one view, then that request's branches;
 * paragraph "Shared branch passes": all requests of a pass in one forward).
 *
 *   n_requests     >= 0
 *   view_len       host [n_requests]: view tokens; 0 marks a shard request
 *                  whose view was scored earlier: its branches start from
 *                  ext_state row e, e counting shard requests in order
 *   branch_count   host [n_requests]: branches of each request (>= 0; a
 *                  request needs a view or at least one branch)
 *   branch_len     host [sum(branch_count)]: branch lengths (>= 1) in request
 *                  order
 *   chunk, block_chunks   as for la_plan_segments
 *   seg_offsets    host [n_segments + 1] or NULL
 *   branch_parent  host [n_segments] or NULL
 *   view_ordinal   host [n_segments] or NULL
 *   plan           host [plan_words] or NULL
 *   info           host, required
 * Segment order: request by request, the view then its branches.  Call with
 * all outputs NULL to learn the sizes (info->n_segments, info->plan_words),
 * then again with the same arguments and buffers of those sizes.
 * Errors: LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED.  Outputs are written only
 * on success.
 */
la_status la_pack_pass(int32_t n_requests, const int32_t* view_len,
                       const int32_t* branch_count, const int32_t* branch_len,
                       int32_t chunk, int32_t block_chunks, int32_t* seg_offsets,
                       int32_t* branch_parent, int32_t* view_ordinal,
                       int32_t* plan, la_pass_info* info);

/*
 * la_pack_pass_ext -- la_pack_pass where each shard request names the
 * ext_state row its branches start from (a row of a view-state cache pool,
 * see la_cache_* below; section "Long Requests").
 *
 *   ext_row        host [n_requests] or NULL: for a request with view_len 0,
 *                  the ext_state row (0 <= row <= 2^30) its branches start
 *                  from; entries of other requests are ignored.  NULL gives
 *                  la_pack_pass (shard requests take rows 0, 1, ... in order).
 * info->n_ext is one past the largest row used.  Other arguments, outputs and
 * errors as la_pack_pass.
 */
la_status la_pack_pass_ext(int32_t n_requests, const int32_t* view_len,
                           const int32_t* branch_count, const int32_t* branch_len,
                           const int32_t* ext_row, int32_t chunk, int32_t block_chunks,
                           int32_t* seg_offsets, int32_t* branch_parent,
                           int32_t* view_ordinal, int32_t* plan, la_pass_info* info);

/*
 * la_scan_workspace_size -- bytes of device workspace la_scan_packed needs:
 * a 256-byte header (a sticky status word, see la_scan_status, and the
 * single-launch form's counters) plus the block states (one fp32 d_k x d_v
 * state per block and head; the piece path, d = 64 with bf16 inputs, also
 * keeps a flag and an inclusive prefix per block and head for its
 * single-launch form).  The same size serves every form of a pass.
 * Errors: LA_ERR_INVALID_ARG (NULL), LA_ERR_UNSUPPORTED (shape/dtype).
 */
la_status la_scan_workspace_size(const la_pass_info* info, int32_t H, int32_t d_k,
                                 int32_t d_v, la_dtype dtype, size_t* bytes);

/*
 * la_scan_packed -- the scan of one packed pass on `stream` (section
 * "Kernels", paragraph "One scan per pass": one scan covers every view of the
 * pass).  The arithmetic, per head: the block states sum_t k_t^T v_t (MFMA),
 * their prefix within each segment (a view's total is final_state), and per
 * chunk o = q S_in + (causal (q k^T)) v carrying S; branch blocks start from
 * their view's total (the same bits as its final_state row) or from
 * ext_state.  It runs in one of three forms, all giving the same bits:
 *   three launches  block states, prefix, outputs (the page's structure);
 *   two launches    block states, then outputs whose workgroups sum the
 *                   states they need themselves (no prefix launch);
 *   one launch      d = 64 with bf16 inputs only: each workgroup computes
 *                   its block's state, obtains the prefix from the
 *                   workgroups before it in the same launch, and computes its
 *                   outputs from the k and v it has already read, so k and v
 *                   cross HBM once.
 * The library picks one launch for d = 64 with bf16 inputs, otherwise two
 * launches for passes whose block states are few (la_pass_info.
 * fused_slot_reads x H x d_k x d_v x 4 bytes up to 128 MiB) and three
 * otherwise; la_scan_launches reports the choice and la_scan_packed_stages
 * can force a form.
 *
 *   q, k           device [T][H][d_k], dtype
 *   v              device [T][H][d_v], dtype
 *   dtype          LA_F32, LA_F32_SPLIT (both fp32 tensors) or LA_BF16
 *   H              heads >= 1
 *   d_k, d_v       head dims; d_k == d_v, 64 or 128
 *   info           host, from the planner that built `plan` (unedited)
 *   plan           device [info->plan_words] int32, a copy of the plan (a
 *                  kernel may read its work record together with the
 *                  header check, so all info->plan_words words must be
 *                  readable even when the plan is another pass's)
 *   ext_state      device [n_ext][H][d_k][d_v] fp32 or NULL when the pass has
 *                  no shard branches (info->n_ext == 0); must not overlap
 *                  final_state
 *   n_ext          rows of ext_state (>= info->n_ext)
 *   out            device [T][H][d_v], dtype: fully overwritten
 *   final_state    device [info->n_views][H][d_k][d_v] fp32, row-major
 *                  (d_v fastest): fully overwritten; NULL iff n_views == 0
 *   workspace      device, >= la_scan_workspace_size bytes, zero-filled
 *                  before its first use (the single-launch form keeps its
 *                  counters and flags there and leaves them zero after every
 *                  pass; fill it with zeros again after an error)
 *   stream         hipStream_t as void*
 * Accumulation is fp32; bf16 outputs are rounded to nearest even.  A pass is
 * idempotent: it reads only its inputs and overwrites all outputs.  Calls
 * that share a workspace must be ordered on one stream.
 * Errors (all detected on the host before anything is enqueued; outputs are
 * then untouched): LA_ERR_INVALID_ARG for NULL or misaligned pointers (q, k,
 * v, out 16-byte aligned; states and plan 4-byte; workspace 16-byte), H < 1,
 * n_ext < info->n_ext, ext_state overlapping final_state, an info whose
 * fields no longer match its checksum, or sizes past the 32-bit dispatch and
 * buffer limits; LA_ERR_UNSUPPORTED for other dtypes, head dims or chunk
 * sizes; LA_ERR_WORKSPACE for a missing or short workspace; LA_ERR_HIP if a
 * launch fails.  Found on the device (recorded in the workspace's status
 * word, see la_scan_status): LA_ERR_PLAN when the device plan is not the one
 * `info` describes (the kernels then do no work), LA_ERR_TIMEOUT when a wait
 * of the single-launch form gave up (its outputs are then not valid).
 */
la_status la_scan_packed(const void* q, const void* k, const void* v, la_dtype dtype,
                         int32_t H, int32_t d_k, int32_t d_v, const la_pass_info* info,
                         const int32_t* plan, const float* ext_state, int32_t n_ext,
                         void* out, float* final_state, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * la_scan_launches -- the form la_scan_packed picks for a pass with these
 * head dims and dtype: 1, 2 or 3 launches, written to *n_launches.  Host only.
 * Errors: LA_ERR_INVALID_ARG (NULL, H < 1), LA_ERR_UNSUPPORTED (head dims).
 */
la_status la_scan_launches(const la_pass_info* info, int32_t H, int32_t d_k, int32_t d_v,
                           la_dtype dtype, int32_t* n_launches);

/*
 * la_scan_status -- reads the sticky status word of a workspace after the
 * passes enqueued on `stream` (synchronises the stream): LA_OK, or an error
 * the kernels recorded (LA_ERR_PLAN, LA_ERR_TIMEOUT; several may be or-ed).
 * clear != 0 resets the word to zero afterwards.
 * Errors: LA_ERR_INVALID_ARG (NULL, workspace shorter than its header),
 * LA_ERR_HIP.
 */
la_status la_scan_status(const void* workspace, size_t workspace_bytes, int32_t* status,
                         int32_t clear, void* stream);

/* Launch selection bits for la_scan_packed_stages. */
#define LA_STAGE_STATES 1     /* launch 1: per-block states          */
#define LA_STAGE_PREFIX 2     /* launch 2: segmented prefix          */
#define LA_STAGE_OUTPUT 4     /* launch 3: chunk outputs             */
#define LA_STAGE_ALL 7
/* Form of the scan, for la_scan_packed_stages (at most one of the three;
 * with none the library picks the form from the pass shape). */
#define LA_FORM_TWO_LAUNCH 8    /* no prefix launch: each output workgroup sums
                                   the block states it needs itself        */
#define LA_FORM_THREE_LAUNCH 16 /* the prefix launch runs between 1 and 3   */
#define LA_FORM_ONE_LAUNCH 32   /* single launch (d = 64, bf16 only); any
                                   LA_STAGE_* bit runs the whole pass      */
/* Test aid for the single-launch form: every wait gives up after a few polls
 * (LA_ERR_TIMEOUT is recorded, the outputs are not valid, every kernel still
 * exits normally). */
#define LA_DEBUG_FORCE_TIMEOUT 64
/* Test aid for the single-launch form: workgroups take their work in ticket
 * order even when the whole launch fits on the GPU at once (the library
 * takes tickets only when it does not). */
#define LA_DEBUG_ORDERED 128

/*
 * la_scan_packed_stages -- la_scan_packed restricted to the launches whose
 * bits are set in `stages` (LA_STAGE_*), with the same arguments and checks.
 * For profiling one launch in isolation.  Launch 2 rewrites the workspace in
 * place, so it must follow a launch 1 on the same buffers; launch 3 only
 * reads the workspace (and ext_state), so after one complete pass it may be
 * repeated alone and produces the same out.  One of the LA_FORM_* bits may be
 * or-ed in to force the form (in the two-launch form the LA_STAGE_PREFIX bit
 * does nothing); every call on one workspace must use the same form.
 * la_scan_packed(...) is la_scan_packed_stages(LA_STAGE_ALL, ...).
 * Errors: as la_scan_packed (LA_ERR_INVALID_ARG also for ext_state overlapping
 * final_state), plus LA_ERR_INVALID_ARG when no LA_STAGE_* bit is set, an
 * unknown bit is set, or more than one LA_FORM_* bit is set, and
 * LA_ERR_UNSUPPORTED for LA_FORM_ONE_LAUNCH, LA_DEBUG_FORCE_TIMEOUT or
 * LA_DEBUG_ORDERED outside the piece path.
 */
la_status la_scan_packed_stages(int32_t stages, const void* q, const void* k, const void* v,
                                la_dtype dtype, int32_t H, int32_t d_k, int32_t d_v,
                                const la_pass_info* info, const int32_t* plan,
                                const float* ext_state, int32_t n_ext, void* out,
                                float* final_state, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * la_export_view_state -- copy one view's final state, for a branch shard
 * that starts from the cached view (section "Long Requests").
 *   final_state  device [n_views][H][d_k][d_v] fp32
 *   view_row     0 <= view_row < n_views
 *   dst          device [H][d_k][d_v] fp32 (may be a row of an ext_state
 *                array); must not overlap the source row
 * Errors: LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_HIP.
 */
la_status la_export_view_state(const float* final_state, int32_t view_row,
                               int32_t n_views, int32_t H, int32_t d_k, int32_t d_v,
                               float* dst, void* stream);

/*
 * la_export_view_kv -- copy a view's keys and values (tokens tok0 ..
 * tok0 + n_tok - 1 of a pass) into a cache pool, for the softmax-attention
 * layers of later branch shards (section "Long Requests": nodes cache the
 * view's linear-attention state and the K/V of its softmax layers).
 *   k, v           device [n_tokens][H][d] (dtype LA_BF16 or LA_F32)
 *   dst_k, dst_v   device [n_tok][H][d] each (e.g. a pool row's region); none
 *                  of the four ranges may overlap another
 * Errors: LA_ERR_INVALID_ARG (range, NULL, alignment, overlap),
 * LA_ERR_UNSUPPORTED (dtype, d), LA_ERR_HIP.
 */
la_status la_export_view_kv(const void* k, const void* v, la_dtype dtype, int32_t n_tokens,
                            int32_t H, int32_t d, int32_t tok0, int32_t n_tok, void* dst_k,
                            void* dst_v, void* stream);

/*
 * Tree-masked softmax attention over a packed pass -- the other layer type of
 * the pass (section "The Workload": Span-1 is mostly linear attention with a
 * few softmax-attention layers; branches attend to their view, never to each
 * other; section "Long Requests": a branch shard attends to its view's
 * cached K/V).  Per head, for every token t:
 *
 *     o_t = sum_{u in A(t)} softmax_u(scale * q_t . k_u) v_u
 *
 * where A(t) is t's own segment up to and including t, plus every token of
 * the parent view for a branch.  A shard branch (parent -2 - e) takes its
 * view's keys and values from external arrays instead (the cached view K/V).
 *
 * la_attn_plan -- host: one work item per (segment, 64-token query block).
 *   n_segments, seg_offsets, branch_parent   the segment table, as for
 *                    la_plan_segments (parents >= 0 must be views; -2 - e
 *                    names external view e)
 *   n_ext            external views (>= 0)
 *   ext_len          host [n_ext]: tokens of each external view (>= 1); the
 *                    views are concatenated in ext_k / ext_v in this order
 *   items            host [*n_items][LA_ATTN_ITEM_WORDS] or NULL (size query;
 *                    fill with a second call on the same arguments)
 *   n_items          host, required: number of items
 * Item layout: {q0, nq, seg0, view0, view_len, view_src, 0, 0}: queries
 * q0 .. q0+nq-1 (nq <= LA_CHUNK) of the segment starting at seg0, whose
 * extra keys are tokens view0 .. view0+view_len-1 of the pass (view_src
 * LA_ATTN_PACKED_VIEW), of ext_k / ext_v (LA_ATTN_EXT_VIEW), or none
 * (LA_ATTN_NO_VIEW).  Items are grouped by the view whose keys they read
 * (a view's query blocks with those of its branches; the branches of one
 * external view form one group); groups go in order of their longest key
 * range (view tokens plus own tokens up to the block's end), ties by the
 * view's segment index, external views after the pass's views, and items
 * within a group longest key range first (ties in table order).
 * Errors: LA_ERR_INVALID_ARG (bad table, parent or length).
 *
 * la_attn_plan_ext -- la_attn_plan where external view e is tokens
 * ext_start[e] .. ext_start[e] + ext_len[e] - 1 of arrays holding ext_tokens
 * token rows (for a pool of cached view K/V: one region per cache row), or,
 * with ext_start NULL, concatenated in order from row 0.
 *   ext_start      host [n_ext] (>= 0) or NULL
 *   ext_tokens     token rows of ext_k / ext_v; every view must lie inside
 * Errors: as la_attn_plan, and LA_ERR_INVALID_ARG for a view outside
 * ext_tokens.  la_attn_packed's n_ext_tokens is then ext_tokens.
 *
 * la_attn_packed -- device: the attention of the pass on `stream`, one
 * workgroup per (item, head): online softmax over 64-key blocks (bf16 MFMA
 * for q.k and p.v, fp32 scores, running max and sums), out rounded to bf16.
 *   q, k, v        device [n_tokens][H][d] bf16 (dtype must be LA_BF16)
 *   d_k, d_v       equal, 64 or 128
 *   scale          score scale, finite and > 0 (e.g. 1/sqrt(d) if k is not
 *                  pre-scaled)
 *   items          device [n_items][LA_ATTN_ITEM_WORDS] int32, a copy of the
 *                  la_attn_plan output for this segment table
 *   ext_k, ext_v   device [n_ext_tokens][H][d] bf16, or NULL if no item
 *                  reads an external view
 *   out            device [n_tokens][H][d_v] bf16: fully overwritten
 * Errors: LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED (dtype, dims), LA_ERR_HIP.
 * The items are trusted (build them with la_attn_plan).
 */
#define LA_ATTN_ITEM_WORDS 8
#define LA_ATTN_NO_VIEW 0
#define LA_ATTN_PACKED_VIEW 1
#define LA_ATTN_EXT_VIEW 2
la_status la_attn_plan(int32_t n_segments, const int32_t* seg_offsets,
                       const int32_t* branch_parent, int32_t n_ext, const int32_t* ext_len,
                       int32_t* items, int32_t* n_items);
la_status la_attn_plan_ext(int32_t n_segments, const int32_t* seg_offsets,
                           const int32_t* branch_parent, int32_t n_ext, const int32_t* ext_len,
                           const int32_t* ext_start, int32_t ext_tokens, int32_t* items,
                           int32_t* n_items);
la_status la_attn_packed(const void* q, const void* k, const void* v, la_dtype dtype, int32_t H,
                         int32_t d_k, int32_t d_v, float scale, const int32_t* items,
                         int32_t n_items, int32_t n_tokens, const void* ext_k,
                         const void* ext_v, int32_t n_ext_tokens, void* out, void* stream);

/*
 * View-state cache directory (section "Long Requests": nodes cache the
 * linear-attention state of recent views so that a branch shard does not
 * recompute its view).  The states live in a caller-owned device pool
 * [capacity][H][d_k][d_v] fp32, which a shard pass uses directly as its
 * ext_state; the directory, a host object, maps view ids (>= 0) to pool rows
 * with least-recently-used eviction.  Typical use:
 *   miss:  la_cache_reserve(view) -> row; run a pass with the view;
 *          la_export_view_state(final_state, view_row, ..., pool + row*H*d*d)
 *   hit:   la_cache_lookup(view) -> row; la_pack_pass_ext with ext_row = row
 *          for the shard request; la_scan_packed(..., ext_state = pool, ...)
 * Device work that reads or writes a row is ordered by the caller's stream: an
 * export into a reused row must be enqueued after every pass that read the
 * evicted view's state, which holds automatically on one stream.  The
 * directory is not thread-safe.
 *
 * la_cache_create   capacity rows (1 .. 2^30); *cache receives the directory
 * la_cache_destroy  frees the directory (not the pool)
 * la_cache_lookup   *row = the view's row (it becomes most recent), or -1
 * la_cache_reserve  *row = a row for view_id: its own if cached, else a free
 *                   row, else the least recently used row, whose view is
 *                   evicted (*evicted_id = its id, or -1; evicted_id may be
 *                   NULL).  The view becomes most recent.
 * la_cache_erase    forget a view (no-op if absent); its row becomes free
 * la_cache_count    *n = views held
 * Errors: LA_ERR_INVALID_ARG for NULL pointers, negative ids, bad capacity.
 */
typedef struct la_state_cache la_state_cache;
la_status la_cache_create(int32_t capacity, la_state_cache** cache);
la_status la_cache_destroy(la_state_cache* cache);
la_status la_cache_lookup(la_state_cache* cache, int64_t view_id, int32_t* row);
la_status la_cache_reserve(la_state_cache* cache, int64_t view_id, int32_t* row,
                           int64_t* evicted_id);
la_status la_cache_erase(la_state_cache* cache, int64_t view_id);
la_status la_cache_count(const la_state_cache* cache, int32_t* n);

/*
 * la_scan_packed_noalloc -- la_scan_packed for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the workspace is taken from an array the library
 * holds in device memory, LA_NOALLOC_SCRATCH_BYTES bytes per GPU, resident
 * from the first call on that GPU until the process ends.  Nothing is
 * allocated and no allocating routine is called; the caller still passes the
 * inputs and outputs.
 *   Arguments, layouts and results as la_scan_packed, without workspace and
 *   workspace_bytes.  The results are those of la_scan_packed (the same
 *   kernels run on the same arguments).
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's contents: calls that may overlap on one GPU (different streams, or
 * graph replays running concurrently) race and must be ordered by the
 * caller.  The first call on a GPU also clears the start of the array (one
 * small kernel on `stream`).
 * Errors: as la_scan_packed, plus LA_ERR_TOO_LARGE when the pass needs more
 * than LA_NOALLOC_SCRATCH_BYTES of workspace (la_scan_workspace_size), and
 * LA_ERR_HIP when the array's device address cannot be obtained.
 */
#define LA_NOALLOC_SCRATCH_BYTES (64u << 20)
la_status la_scan_packed_noalloc(const void* q, const void* k, const void* v, la_dtype dtype,
                                 int32_t H, int32_t d_k, int32_t d_v,
                                 const la_pass_info* info, const int32_t* plan,
                                 const float* ext_state, int32_t n_ext, void* out,
                                 float* final_state, void* stream);

/* Static text for a status code. */
const char* la_status_string(la_status status);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
