"""The entry point that allocates nothing (la_scan_packed_noalloc), called
through the C ABI: its outputs equal those of la_scan_packed with a
caller-owned workspace, bit for bit (the same kernels run on the same
arguments), on two calls in a row, the second smaller than the first, and
both lie within the bf16 tolerance of the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import chunked_linear_attention_packed_amd as la
import oracle
import synth


def _call_noalloc(lib, q, k, v, plan, out, fin, ext=None):
    H, d = q.shape[1], q.shape[2]
    dev = q.device
    dplan = plan.device_plan(dev)
    stream = torch.cuda.current_stream(dev)
    return lib.la_scan_packed_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), la._dtype_code(q), H, d, d, ctypes.byref(plan.info),
        ctypes.c_void_p(dplan.data_ptr()),
        None if ext is None else ctypes.c_void_p(ext.data_ptr()),
        0 if ext is None else ext.shape[0], ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(fin.data_ptr()) if fin.numel() else None,
        ctypes.c_void_p(stream.cuda_stream))


@pytest.mark.gpu
def test_noalloc_equals_workspace_entry_point_twice():
    lib = la.load_library()
    dev = torch.device("cuda:0")
    # first the larger pass, then a smaller one on the same scratch array
    cases = [([1500, 300], [6, 3], [48, 1, 100, 33, 64, 65, 7, 128, 90], 8, "bf16"),
             ([200], [2], [16, 70], 4, "bf16")]
    for i, (vl, bc, bl, H, dt) in enumerate(cases):
        print(f"noalloc case {i}: views {vl} branches {bl} H {H}", flush=True)
        plan = la.pack(vl, bc, bl, heads=H)
        so, bp = plan.seg_offsets, plan.branch_parent
        q, k, v = synth.draw_qkv(np.random.default_rng(40 + i), int(so[-1]), H, 64, dt)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        ref_o, ref_f = la.scan_packed(qd, kd, vd, plan)
        out = torch.full_like(ref_o, float("nan"))
        fin = torch.full_like(ref_f, float("nan"))
        st = _call_noalloc(lib, qd, kd, vd, plan, out, fin)
        torch.cuda.synchronize()
        assert st == la.LA_OK, lib.la_status_string(st)
        assert torch.equal(out, ref_o)
        assert torch.equal(fin, ref_f)
        oo, of = oracle.scan_recurrence(q, k, v, so, bp)
        assert oracle.row_rel_err(out.cpu(), oo) <= 2e-2
        assert oracle.state_rel_err(fin.cpu(), of) <= 2e-2
