// Internal interface between the scan entry points (scan.hip) and the piece
// path (piece.hip): the d = 64, bf16 scan whose waves each own a piece of
// LA_PIECE_CHUNKS consecutive chunks.  Not part of the public ABI.
#ifndef LINATTN_PIECE_H
#define LINATTN_PIECE_H

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "linattn.h"

namespace piece {

// Workspace header (every form of the piece path; the first 256 bytes):
// word kStatusWord is a sticky status (0 or the last error the kernels met,
// see la_scan_status); the single-launch form keeps its ticket and retire
// counters in the next words.  The single-launch form needs the header and
// the flag region zero before its first pass and leaves them zero after
// every pass.
constexpr size_t kHeaderBytes = 256;
constexpr int kStatusWord = 0;
constexpr int kTicketWord = 2;
constexpr int kRetireWord = 3;

// Bytes of workspace the piece path needs for a pass (all its forms).
size_t workspace_bytes(const la_pass_info& info, int32_t H);

// True when the piece path runs this pass (d = 64, bf16).
inline bool applies(int32_t d, la_dtype dtype) { return d == 64 && dtype == LA_BF16; }

// Enqueues the launches of `stages` (LA_STAGE_* bits) in form `form`
// (1, 2 or 3 launches).  Arguments are validated by the caller.  In the
// single-launch form, `ordered` makes the workgroups take tickets even when
// the whole launch fits on the device at once.
la_status launch(int32_t stages, int form, const void* q, const void* k, const void* v,
                 int32_t H, const la_pass_info& info, const int32_t* plan,
                 const float* ext_state, void* out, float* final_state, void* workspace,
                 hipStream_t stream, int32_t spin_limit, bool force_timeout, bool ordered);

// The prefix launch of the shared scan code over the piece path's slots
// (defined in scan.hip, which holds the prefix kernel).
la_status launch_prefix(const int32_t* scans, int32_t n_scan, float* slots, float* final_state,
                        int32_t H, hipStream_t st, const int32_t* plan, int* hdr, int hash);

}  // namespace piece

#endif  // LINATTN_PIECE_H
