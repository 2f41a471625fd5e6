"""Python binding of liblinattn.so: the packed chunked causal linear-attention
scan for MI355X (gfx950).

Argument marshalling only.  Every step of the scan runs in the HIP library;
PyTorch supplies device memory and the stream.  There is no fallback: if the
library is missing or was built without the GPU code, calls raise.

Source of the method: "Serving 0.88M TPS from Two RTXs and Mac Minis",
sections "The Workload", "Kernels" and "Long Requests".

    plan = pack(view_len, branch_count, branch_len, heads=H)
    out, final_state = scan_packed(q, k, v, plan)
    export_view_state(final_state, view_row, dst)

Branch shards (section "Long Requests"): a ViewStateCache keeps view states
in a device pool; a shard request (view length 0) packed with
ext_row=[cache row] runs from the cached state:

    cache = ViewStateCache(capacity, H, d, device)
    row = cache.store(view_id, final_state, view_row)         # after the view
    plan = pack([0], [n], lens, heads=H, ext_row=[cache.lookup(view_id)])
    out, _ = scan_packed(q, k, v, plan, ext_state=cache.pool)
"""
import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = ["LinAttnError", "PassInfo", "PassPlan", "pack", "plan_segments",
           "choose_block_chunks", "workspace_size", "new_workspace", "scan_launches",
           "scan_status", "scan_packed",
           "export_view_state", "ViewStateCache", "AttnPlan", "attn_plan", "attn_packed",
           "library_path", "load_library", "CHUNK"]

CHUNK = 64
(LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE, LA_ERR_HIP,
 LA_ERR_TOO_LARGE, LA_ERR_PLAN, LA_ERR_TIMEOUT) = range(8)
NOALLOC_SCRATCH_BYTES = 64 << 20
LA_F32, LA_BF16, LA_F32_SPLIT = 0, 1, 2
LA_ATTN_NO_VIEW, LA_ATTN_PACKED_VIEW, LA_ATTN_EXT_VIEW = 0, 1, 2
STAGE_STATES, STAGE_PREFIX, STAGE_OUTPUT, STAGE_ALL = 1, 2, 4, 7
FORM_TWO_LAUNCH, FORM_THREE_LAUNCH, FORM_ONE_LAUNCH = 8, 16, 32
DEBUG_FORCE_TIMEOUT = 64
DEBUG_ORDERED = 128
_FORMS = {None: 0, "auto": 0, "one": FORM_ONE_LAUNCH, "two": FORM_TWO_LAUNCH,
          "three": FORM_THREE_LAUNCH}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.path.join(_HERE, "liblinattn.so")


class LinAttnError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class PassInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_requests", "n_segments", "n_views", "n_branches", "n_ext", "n_tokens", "chunk",
        "block_chunks", "n_chunks", "n_view_chunks", "n_blocks", "n_delta", "n_scan",
        "plan_words", "max_seg_tokens", "fused_slot_reads", "piece_blocks", "piece_items",
        "piece_block_items", "piece_slots", "piece_scans", "plan_hash", "info_check")] + [
        ("reserved", ctypes.c_int32 * 1)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_ if n != "reserved"}


_lib = None
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)


def load_library():
    """Load liblinattn.so once.  Raises if it is absent: nothing here runs
    the scan any other way."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with "
            "`python -m chunked_linear_attention_packed_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    lib.la_pack_pass.argtypes = [ctypes.c_int32, _I32P, _I32P, _I32P, ctypes.c_int32,
                                 ctypes.c_int32, _I32P, _I32P, _I32P, _I32P,
                                 ctypes.POINTER(PassInfo)]
    lib.la_plan_segments.argtypes = [ctypes.c_int32, _I32P, _I32P, ctypes.c_int32,
                                     ctypes.c_int32, _I32P, _I32P, ctypes.POINTER(PassInfo)]
    lib.la_scan_workspace_size.argtypes = [ctypes.POINTER(PassInfo), ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_size_t)]
    lib.la_scan_packed.argtypes = [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.POINTER(PassInfo), _P, _P,
                                   ctypes.c_int32, _P, _P, _P, ctypes.c_size_t, _P]
    lib.la_scan_packed_stages.argtypes = [ctypes.c_int32] + lib.la_scan_packed.argtypes
    lib.la_scan_packed_noalloc.argtypes = lib.la_scan_packed.argtypes[:13] + [_P]
    lib.la_scan_launches.argtypes = [ctypes.POINTER(PassInfo), ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, _I32P]
    lib.la_scan_status.argtypes = [_P, ctypes.c_size_t, _I32P, ctypes.c_int32, _P]
    lib.la_info_checksum.argtypes = [ctypes.POINTER(PassInfo)]
    lib.la_info_checksum.restype = ctypes.c_uint32
    lib.la_choose_block_chunks.argtypes = [ctypes.c_int32, _I32P, _I32P, ctypes.c_int32, _I32P]
    lib.la_export_view_state.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, _P, _P]
    lib.la_pack_pass_ext.argtypes = [ctypes.c_int32, _I32P, _I32P, _I32P, _I32P,
                                     ctypes.c_int32, ctypes.c_int32, _I32P, _I32P, _I32P,
                                     _I32P, ctypes.POINTER(PassInfo)]
    lib.la_cache_create.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
    lib.la_cache_destroy.argtypes = [ctypes.c_void_p]
    lib.la_cache_lookup.argtypes = [ctypes.c_void_p, ctypes.c_int64, _I32P]
    lib.la_cache_reserve.argtypes = [ctypes.c_void_p, ctypes.c_int64, _I32P,
                                     ctypes.POINTER(ctypes.c_int64)]
    lib.la_cache_erase.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    lib.la_cache_count.argtypes = [ctypes.c_void_p, _I32P]
    lib.la_attn_plan.argtypes = [ctypes.c_int32, _I32P, _I32P, ctypes.c_int32, _I32P, _I32P,
                                 _I32P]
    lib.la_attn_plan_ext.argtypes = [ctypes.c_int32, _I32P, _I32P, ctypes.c_int32, _I32P, _I32P,
                                     ctypes.c_int32, _I32P, _I32P]
    lib.la_export_view_kv.argtypes = [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
    lib.la_attn_packed.argtypes = [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_float, _P, ctypes.c_int32,
                                   ctypes.c_int32, _P, _P, ctypes.c_int32, _P, _P]
    lib.la_status_string.argtypes = [ctypes.c_int32]
    lib.la_status_string.restype = ctypes.c_char_p
    for fn in ("la_pack_pass", "la_pack_pass_ext", "la_plan_segments",
               "la_scan_workspace_size", "la_scan_packed", "la_scan_packed_stages",
               "la_scan_packed_noalloc", "la_scan_status",
               "la_scan_launches", "la_choose_block_chunks", "la_export_view_state", "la_cache_create", "la_cache_destroy",
               "la_cache_lookup", "la_cache_reserve", "la_cache_erase", "la_cache_count",
               "la_attn_plan", "la_attn_plan_ext", "la_attn_packed", "la_export_view_kv"):
        getattr(lib, fn).restype = ctypes.c_int32
    _lib = lib
    return lib


def _check(fn, status):
    if status != LA_OK:
        msg = load_library().la_status_string(status).decode()
        raise LinAttnError(fn, status, msg)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a):
    return a.ctypes.data_as(_I32P) if a is not None and a.size else None


@dataclass
class PassPlan:
    """Host result of packing: segment table, info and the device plan."""
    info: PassInfo
    seg_offsets: np.ndarray
    branch_parent: np.ndarray
    view_ordinal: np.ndarray
    plan: np.ndarray
    _dev: dict = field(default_factory=dict, repr=False)

    def device_plan(self, device):
        """The plan as an int32 tensor on `device`, uploaded once."""
        import torch
        key = str(torch.device(device))
        if key not in self._dev:
            self._dev[key] = torch.from_numpy(self.plan).to(device)
        return self._dev[key]


def choose_block_chunks(seg_offsets, branch_parent, heads):
    """Work-block size for a segment table and H heads, from the library's
    rule (la_choose_block_chunks)."""
    lib = load_library()
    so, bp = _i32(seg_offsets), _i32(branch_parent)
    g = ctypes.c_int32()
    _check("la_choose_block_chunks",
           lib.la_choose_block_chunks(len(bp), _ptr(so), _ptr(bp), heads, ctypes.byref(g)))
    return g.value


def pack(view_len, branch_count, branch_len, heads=16, block_chunks=None, chunk=CHUNK,
         ext_row=None):
    """Request shapes -> PassPlan via la_pack_pass_ext (view then branches per
    request; view length 0 marks a shard request seeded from ext_state: row
    ext_row[r] if given, else the next row in order)."""
    lib = load_library()
    vl, bc, bl = _i32(view_len), _i32(branch_count), _i32(branch_len)
    er = None if ext_row is None else _i32(ext_row)
    if er is not None and len(er) != len(vl):
        raise ValueError("ext_row needs one entry per request")
    # the library reads exactly len(view_len) counts and sum(branch_count)
    # branch lengths
    if len(bc) != len(vl):
        raise ValueError("branch_count needs one entry per request")
    if len(bl) != int(np.sum(np.maximum(bc, 0), dtype=np.int64)):
        raise ValueError("branch_len needs sum(branch_count) entries")
    info = PassInfo()
    if block_chunks is None:   # the segment table first, then the library's block size
        _check("la_pack_pass", lib.la_pack_pass_ext(len(vl), _ptr(vl), _ptr(bc), _ptr(bl),
                                                    _ptr(er), chunk, 1, None, None, None, None,
                                                    ctypes.byref(info)))
        so = np.zeros(info.n_segments + 1, dtype=np.int32)
        bp = np.zeros(info.n_segments, dtype=np.int32)
        _check("la_pack_pass", lib.la_pack_pass_ext(len(vl), _ptr(vl), _ptr(bc), _ptr(bl),
                                                    _ptr(er), chunk, 1,
                                                    so.ctypes.data_as(_I32P), _ptr(bp), None,
                                                    None, ctypes.byref(info)))
        block_chunks = choose_block_chunks(so, bp, heads)
    _check("la_pack_pass", lib.la_pack_pass_ext(len(vl), _ptr(vl), _ptr(bc), _ptr(bl),
                                                _ptr(er), chunk, block_chunks, None, None,
                                                None, None, ctypes.byref(info)))
    so = np.zeros(info.n_segments + 1, dtype=np.int32)
    bp = np.zeros(info.n_segments, dtype=np.int32)
    vo = np.zeros(info.n_segments, dtype=np.int32)
    plan = np.zeros(info.plan_words, dtype=np.int32)
    _check("la_pack_pass", lib.la_pack_pass_ext(len(vl), _ptr(vl), _ptr(bc), _ptr(bl),
                                                _ptr(er), chunk, block_chunks,
                                                so.ctypes.data_as(_I32P), _ptr(bp), _ptr(vo),
                                                _ptr(plan), ctypes.byref(info)))
    return PassPlan(info, so, bp, vo, plan)


def plan_segments(seg_offsets, branch_parent, heads=16, block_chunks=None, chunk=CHUNK):
    """Segment table (any order whose parents are views) -> PassPlan."""
    lib = load_library()
    so, bp = _i32(seg_offsets), _i32(branch_parent)
    if block_chunks is None:
        block_chunks = choose_block_chunks(so, bp, heads)
    info = PassInfo()
    _check("la_plan_segments", lib.la_plan_segments(len(bp), _ptr(so), _ptr(bp), chunk,
                                                    block_chunks, None, None,
                                                    ctypes.byref(info)))
    vo = np.zeros(info.n_segments, dtype=np.int32)
    plan = np.zeros(info.plan_words, dtype=np.int32)
    _check("la_plan_segments", lib.la_plan_segments(len(bp), _ptr(so), _ptr(bp), chunk,
                                                    block_chunks, _ptr(vo), _ptr(plan),
                                                    ctypes.byref(info)))
    return PassPlan(info, so, bp, vo, plan)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def workspace_size(plan, heads, d, dtype):
    lib = load_library()
    n = ctypes.c_size_t()
    code = dtype if isinstance(dtype, int) else _dtype_code_from_torch(dtype)
    _check("la_scan_workspace_size",
           lib.la_scan_workspace_size(ctypes.byref(plan.info), heads, d, d, code,
                                      ctypes.byref(n)))
    return n.value


def scan_launches(plan, heads, d, dtype=LA_BF16):
    """Launches scan_packed uses for this pass by default: 1, 2 or 3."""
    lib = load_library()
    n = ctypes.c_int32()
    code = dtype if isinstance(dtype, int) else _dtype_code_from_torch(dtype)
    _check("la_scan_launches",
           lib.la_scan_launches(ctypes.byref(plan.info), heads, d, d, code, ctypes.byref(n)))
    return n.value


def new_workspace(plan, heads, d, dtype, device, stream=None):
    """A zero-filled workspace of the size the pass needs (the single-launch
    form needs its header and flags zero before the first pass)."""
    import torch
    n = max(workspace_size(plan, heads, d, dtype), 256)
    if stream is None:
        return torch.zeros(n, dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.zeros(n, dtype=torch.uint8, device=device)


def scan_status(workspace, clear=False, stream=None):
    """The sticky status word the kernels left in a workspace (0: none; else
    LA_ERR_PLAN / LA_ERR_TIMEOUT bits); synchronises the stream."""
    lib = load_library()
    st = ctypes.c_int32()
    _check("la_scan_status",
           lib.la_scan_status(ctypes.c_void_p(workspace.data_ptr()),
                              workspace.numel() * workspace.element_size(), ctypes.byref(st),
                              1 if clear else 0, _stream_ptr(stream, workspace.device)))
    return st.value


def _dtype_code_from_torch(dt):
    import torch
    return {torch.bfloat16: LA_BF16, torch.float32: LA_F32}[dt]


def _stream_ptr(stream, device):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _alloc(shape, dtype, device, stream):
    """torch.empty on `stream`'s side of the caching allocator: a buffer made
    for work enqueued on a caller-given stream is returned to that stream's
    pool when it is dropped, so no later allocation on another stream can
    reuse it while the work still runs."""
    import torch
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _check_tensor(name, t, shape, dtype, device, min_rows=None):
    """Shape, dtype, device and layout of a caller-supplied buffer; the C ABI
    sees only its address, so a wrong one would be read or written past its
    end."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if min_rows is None:
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    elif t.dim() != len(shape) or tuple(t.shape[1:]) != tuple(shape[1:]) or t.shape[0] < min_rows:
        raise ValueError(f"{name} must have shape [>= {min_rows}, {', '.join(map(str, shape[1:]))}],"
                         f" got {tuple(t.shape)}")


def check_scan_buffers(q, v, info, out=None, final_state=None, ext_state=None, workspace=None,
                       need=0):
    """Validates the caller-supplied buffers of scan_packed against the inputs
    and the pass (any device: also usable on CPU tensors)."""
    import torch
    T, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    if out is not None:
        _check_tensor("out", out, (T, H, dv), q.dtype, dev)
    if final_state is not None:
        _check_tensor("final_state", final_state, (info.n_views, H, dk, dv), torch.float32, dev)
    if ext_state is not None:
        _check_tensor("ext_state", ext_state, (info.n_ext, H, dk, dv), torch.float32, dev,
                      min_rows=info.n_ext)
    elif info.n_ext > 0:
        raise ValueError(f"the pass has shard branches: ext_state needs >= {info.n_ext} rows")
    if workspace is not None:
        if workspace.device != dev:
            raise ValueError(f"workspace must be on {dev}, got {workspace.device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace needs {need} bytes")


def scan_packed(q, k, v, plan, ext_state=None, out=None, final_state=None, workspace=None,
                stream=None, stages=STAGE_ALL, split_fp32=False, form=None):
    """Run the scan on `stream` (default: torch's current stream).

    q, k: [T, H, d] and v: [T, H, d] contiguous CUDA tensors, bf16 or fp32.
    Returns (out [T, H, d] in the input dtype, final_state [n_views, H, d, d]
    fp32).  Pre-allocated out / final_state / workspace tensors are used as
    given (no allocation then); they are checked for shape, dtype, device and
    layout.  Buffers allocated here for work on a caller-given stream come
    from that stream's pool.  `stages` selects launches (STAGE_* bits, see
    la_scan_packed_stages) for profiling; the default runs all of them.  For
    fp32 inputs, split_fp32=True evaluates every product as three bf16 MFMAs
    over hi/lo operand splits (LA_F32_SPLIT) instead of fp32 MFMAs.  `form`
    forces the single-launch ("one": d 64 bf16 only), two-launch ("two": no
    prefix launch) or three-launch ("three") form; None lets the library
    choose.  A caller-given workspace must be zero-filled before its first
    use (new_workspace)."""
    import torch
    lib = load_library()
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k: [T, H, d_k]; v: [T, H, d_v]")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    T, H, dk = q.shape
    dv = v.shape[2]
    info = plan.info
    if T != info.n_tokens:
        raise ValueError(f"q has {T} tokens, the plan {info.n_tokens}")
    code = _dtype_code(q)
    if split_fp32:
        if code != LA_F32:
            raise TypeError("split_fp32 applies to float32 inputs")
        code = LA_F32_SPLIT
    if form not in _FORMS:
        raise ValueError(f"form must be one of {sorted(k for k in _FORMS if k)} or None")
    dev = q.device
    need = workspace_size(plan, H, dk, code)
    check_scan_buffers(q, v, info, out, final_state, ext_state, workspace, need)
    if out is None:
        out = _alloc((T, H, dv), q.dtype, dev, stream)
    if final_state is None:
        final_state = _alloc((info.n_views, H, dk, dv), torch.float32, dev, stream)
    if workspace is None:
        workspace = new_workspace(plan, H, dk, code, dev, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    n_ext = 0
    ext_ptr = None
    if ext_state is not None:
        n_ext = ext_state.shape[0]
        ext_ptr = ctypes.c_void_p(ext_state.data_ptr())
    dplan = plan.device_plan(dev)
    st = lib.la_scan_packed_stages(stages | _FORMS[form], ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                            ctypes.c_void_p(v.data_ptr()), code, H, dk, dv,
                            ctypes.byref(info), ctypes.c_void_p(dplan.data_ptr()), ext_ptr,
                            n_ext, ctypes.c_void_p(out.data_ptr()),
                            ctypes.c_void_p(final_state.data_ptr()) if final_state.numel() else None,
                            ctypes.c_void_p(workspace.data_ptr()), ws_bytes,
                            _stream_ptr(stream, dev))
    _check("la_scan_packed", st)
    return out, final_state


def export_view_state(final_state, view_row, dst=None, stream=None):
    """Copy final_state[view_row] ([H, d, d] fp32) into dst (allocated if
    None) on the device, for a branch shard seeded from the cached view."""
    import torch
    lib = load_library()
    nv, H, dk, dv = final_state.shape
    if final_state.dtype != torch.float32 or not final_state.is_contiguous():
        raise TypeError("final_state must be contiguous float32 [n_views, H, d, d]")
    if dst is None:
        dst = _alloc((H, dk, dv), torch.float32, final_state.device, stream)
    else:
        _check_tensor("dst", dst, (H, dk, dv), torch.float32, final_state.device)
    _check("la_export_view_state",
           lib.la_export_view_state(ctypes.c_void_p(final_state.data_ptr()), view_row, nv, H,
                                    dk, dv, ctypes.c_void_p(dst.data_ptr()),
                                    _stream_ptr(stream, final_state.device)))
    return dst


def export_view_kv(k, v, tok0, n_tok, dst_k, dst_v, stream=None):
    """Copy tokens tok0 .. tok0 + n_tok - 1 of k and v ([T, H, d]) into
    dst_k, dst_v ([n_tok, H, d], e.g. a K/V pool row's region) on the device."""
    lib = load_library()
    if k.dim() != 3 or v.shape != k.shape or k.dtype != v.dtype:
        raise ValueError("k, v: [T, H, d] of one dtype")
    T, H, d = k.shape
    if not (k.is_contiguous() and v.is_contiguous()):
        raise ValueError("k, v must be contiguous")
    for name, t in (("dst_k", dst_k), ("dst_v", dst_v)):
        _check_tensor(name, t, (n_tok, H, d), k.dtype, k.device)
    _check("la_export_view_kv",
           lib.la_export_view_kv(ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                 _dtype_code(k), T, H, d, tok0, n_tok,
                                 ctypes.c_void_p(dst_k.data_ptr()),
                                 ctypes.c_void_p(dst_v.data_ptr()), _stream_ptr(stream, k.device)))


class ViewStateCache:
    """The view cache of a node (section "Long Requests"): for each cached view,
    its linear-attention state and, when kv_tokens > 0, the K/V of its softmax
    layers, in device pools with the library's least-recently-used directory
    (la_cache_*), so branch shards skip their view.

    pool   [capacity, H, d, d] fp32: the ext_state of shard passes (lookup
           gives the row to pass as ext_row);
    kv_k, kv_v   [kv_layers, capacity * kv_tokens, H, d]: row r of the
           directory owns token rows r * kv_tokens .. of each layer; a shard's
           attention names them with kv_extent (ext_start / ext_len of
           attn_plan, ext_tokens = capacity * kv_tokens).

    Device copies go on the caller's stream; not thread-safe."""

    def __init__(self, capacity, heads, d, device="cuda", kv_tokens=0, kv_layers=1,
                 kv_dtype=None):
        import torch
        lib = load_library()
        self._lib = lib
        self._h = ctypes.c_void_p()
        _check("la_cache_create", lib.la_cache_create(capacity, ctypes.byref(self._h)))
        self.capacity, self.heads, self.d = capacity, heads, d
        self.pool = torch.empty((capacity, heads, d, d), dtype=torch.float32, device=device)
        self.kv_tokens, self.kv_layers = int(kv_tokens), int(kv_layers)
        self.kv_k = self.kv_v = None
        if self.kv_tokens > 0:
            shape = (self.kv_layers, capacity * self.kv_tokens, heads, d)
            dt = torch.bfloat16 if kv_dtype is None else kv_dtype
            self.kv_k = torch.empty(shape, dtype=dt, device=device)
            self.kv_v = torch.empty(shape, dtype=dt, device=device)

    @property
    def _kv_len(self):
        """row -> tokens of K/V held in that row's region."""
        return self.__dict__.setdefault("_kv_rows", {})

    def lookup(self, view_id):
        """Pool row holding view_id's state (now most recent), or None."""
        row = ctypes.c_int32()
        _check("la_cache_lookup", self._lib.la_cache_lookup(self._h, view_id, ctypes.byref(row)))
        return None if row.value < 0 else row.value

    def reserve(self, view_id):
        """(row, evicted view id or None): the row to write view_id's state to."""
        row, ev = ctypes.c_int32(), ctypes.c_int64()
        _check("la_cache_reserve", self._lib.la_cache_reserve(self._h, view_id,
                                                              ctypes.byref(row),
                                                              ctypes.byref(ev)))
        self._kv_len.pop(row.value, None)   # the row's K/V, if any, are not view_id's
        return row.value, (None if ev.value < 0 else ev.value)

    def store(self, view_id, final_state, view_row, stream=None, kv=None, view_tok0=0,
              view_tokens=0):
        """Copy final_state[view_row] into view_id's pool row (evicting the
        least recently used view if the pool is full); with kv = [(k, v) per
        softmax layer] ([T, H, d] of the pass that scored the view), also
        copy the view's tokens view_tok0 .. view_tok0 + view_tokens - 1 of
        each layer into the row's K/V region.  Returns the row."""
        if final_state.shape[1:] != self.pool.shape[1:]:
            raise ValueError("final_state rows must be [H, d, d] of this cache")
        if kv is not None:
            if self.kv_k is None:
                raise ValueError("this cache holds no K/V (kv_tokens = 0)")
            if len(kv) != self.kv_layers:
                raise ValueError(f"kv needs {self.kv_layers} (k, v) pairs")
            if not 1 <= view_tokens <= self.kv_tokens:
                raise ValueError(f"view_tokens must be 1 .. {self.kv_tokens}")
        row, _ = self.reserve(view_id)
        export_view_state(final_state, view_row, self.pool[row], stream=stream)
        if kv is not None:
            a = row * self.kv_tokens
            for layer, (k, v) in enumerate(kv):
                export_view_kv(k, v, view_tok0, view_tokens,
                               self.kv_k[layer, a:a + view_tokens],
                               self.kv_v[layer, a:a + view_tokens], stream=stream)
            self._kv_len[row] = int(view_tokens)
        return row

    def kv_extent(self, view_id):
        """(row, first token row, tokens) of view_id's cached K/V in kv_k /
        kv_v, or None (not cached, or cached without K/V).  Marks the view
        most recent."""
        row = self.lookup(view_id)
        if row is None or row not in self._kv_len:
            return None
        return row, row * self.kv_tokens, self._kv_len[row]

    @property
    def kv_pool_tokens(self):
        return self.capacity * self.kv_tokens

    def erase(self, view_id):
        row = self.lookup(view_id)
        _check("la_cache_erase", self._lib.la_cache_erase(self._h, view_id))
        if row is not None:
            self._kv_len.pop(row, None)

    def __len__(self):
        n = ctypes.c_int32()
        _check("la_cache_count", self._lib.la_cache_count(self._h, ctypes.byref(n)))
        return n.value

    def close(self):
        if self._h:
            self._lib.la_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


@dataclass
class AttnPlan:
    """Work items of the tree-masked softmax attention of one segment table
    (la_attn_plan): one per (segment, 64-token query block)."""
    n_tokens: int
    n_ext_tokens: int
    items: np.ndarray            # [n_items, 8] int32
    _dev: dict = field(default_factory=dict, repr=False)

    def device_items(self, device):
        import torch
        key = str(torch.device(device))
        if key not in self._dev:
            self._dev[key] = torch.from_numpy(self.items.reshape(-1)).to(device)
        return self._dev[key]


def attn_plan(seg_offsets, branch_parent, ext_len=None, ext_start=None, ext_tokens=None):
    """Segment table (parents >= 0 are views, -2 - e external view e of
    ext_len[e] tokens) -> AttnPlan.  External views are concatenated in
    ext_k / ext_v, or, with ext_start, view e starts at token row
    ext_start[e] of arrays of ext_tokens rows (a K/V cache pool)."""
    lib = load_library()
    so, bp = _i32(seg_offsets), _i32(branch_parent)
    el = _i32([] if ext_len is None else ext_len)
    if ext_start is None:
        st, n_rows = None, int(el.sum())
    else:
        st = _i32(ext_start)
        if len(st) != len(el) or ext_tokens is None:
            raise ValueError("ext_start needs one entry per external view, and ext_tokens")
        n_rows = int(ext_tokens)
    n = ctypes.c_int32()
    _check("la_attn_plan", lib.la_attn_plan_ext(len(bp), _ptr(so), _ptr(bp), len(el), _ptr(el),
                                                _ptr(st), n_rows, None, ctypes.byref(n)))
    items = np.zeros((n.value, 8), dtype=np.int32)
    _check("la_attn_plan", lib.la_attn_plan_ext(len(bp), _ptr(so), _ptr(bp), len(el), _ptr(el),
                                                _ptr(st), n_rows, _ptr(items), ctypes.byref(n)))
    return AttnPlan(int(so[-1]) if len(so) else 0, n_rows, items)


def attn_packed(q, k, v, plan, scale, ext_k=None, ext_v=None, out=None, stream=None):
    """Tree-masked softmax attention of a packed pass (bf16 q, k, v
    [T, H, d]); ext_k / ext_v [n_ext_tokens, H, d] hold the external views
    that shard branches attend to.  Returns out [T, H, d] bf16."""
    import torch
    lib = load_library()
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v: [T, H, d]")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    T, H, d = q.shape
    if T != plan.n_tokens:
        raise ValueError(f"q has {T} tokens, the plan {plan.n_tokens}")
    n_ext = 0
    ek = ev = None
    if plan.n_ext_tokens:
        if ext_k is None or ext_v is None:
            raise ValueError("the plan reads external views: pass ext_k and ext_v")
        if ext_k.shape != (plan.n_ext_tokens, H, d) or ext_v.shape != ext_k.shape:
            raise ValueError(f"ext_k / ext_v must be [{plan.n_ext_tokens}, {H}, {d}]")
        if ext_k.dtype != q.dtype or ext_v.dtype != q.dtype:
            raise TypeError("ext_k / ext_v must have the dtype of q")
        if not (ext_k.is_contiguous() and ext_v.is_contiguous()):
            raise ValueError("ext_k / ext_v must be contiguous")
        n_ext = plan.n_ext_tokens
        ek, ev = ctypes.c_void_p(ext_k.data_ptr()), ctypes.c_void_p(ext_v.data_ptr())
    if out is None:
        out = torch.empty_like(v)
    items = plan.device_items(q.device)
    _check("la_attn_packed",
           lib.la_attn_packed(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                              ctypes.c_void_p(v.data_ptr()), _dtype_code(q), H, d, d,
                              float(scale), ctypes.c_void_p(items.data_ptr()),
                              len(plan.items), T, ek, ev, n_ext,
                              ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream, q.device)))
    return out
