"""Host checks of the Python binding (no GPU): caller-supplied buffers are
validated before their addresses reach the C ABI, which cannot see their
sizes, and buffers the binding allocates for work on a caller-given stream
are taken from that stream's side of the caching allocator."""
import contextlib

import pytest
import torch

import chunked_linear_attention_packed_amd as la


def _plan():
    # two requests (view 100 + 2 branches, view 70 + 1 branch) and a shard
    # request of one branch seeded from ext_state row 0
    return la.pack([100, 70, 0], [2, 1, 1], [5, 9, 30, 12], heads=2, block_chunks=2)


def _inputs(plan, dtype=torch.bfloat16, d=64):
    T = plan.info.n_tokens
    q = torch.zeros((T, 2, d), dtype=dtype)
    v = torch.zeros((T, 2, d), dtype=dtype)
    return q, v


def test_valid_buffers_pass():
    plan = _plan()
    q, v = _inputs(plan)
    T, H, d = q.shape
    la.check_scan_buffers(q, v, plan.info,
                          out=torch.empty((T, H, d), dtype=q.dtype),
                          final_state=torch.empty((plan.info.n_views, H, d, d)),
                          ext_state=torch.empty((3, H, d, d)),
                          workspace=torch.empty(100, dtype=torch.uint8), need=100)


@pytest.mark.parametrize("case", ["out_dtype", "out_shape", "out_layout", "fin_rows",
                                  "fin_dtype", "ext_rows", "ext_missing", "ext_dims",
                                  "ws_small", "ws_layout"])
def test_bad_buffers_are_rejected(case):
    plan = _plan()
    q, v = _inputs(plan)
    T, H, d = q.shape
    nv = plan.info.n_views
    kw = dict(out=torch.empty((T, H, d), dtype=q.dtype),
              final_state=torch.empty((nv, H, d, d)),
              ext_state=torch.empty((1, H, d, d)),
              workspace=torch.empty(64, dtype=torch.uint8), need=64)
    if case == "out_dtype":
        kw["out"] = torch.empty((T, H, d), dtype=torch.float32)
    elif case == "out_shape":
        kw["out"] = torch.empty((T - 1, H, d), dtype=q.dtype)
    elif case == "out_layout":
        kw["out"] = torch.empty((T, d, H), dtype=q.dtype).transpose(1, 2)
    elif case == "fin_rows":
        kw["final_state"] = torch.empty((nv - 1, H, d, d))
    elif case == "fin_dtype":
        kw["final_state"] = torch.empty((nv, H, d, d), dtype=torch.bfloat16)
    elif case == "ext_rows":
        kw["ext_state"] = torch.empty((0, H, d, d))
    elif case == "ext_missing":
        kw["ext_state"] = None
    elif case == "ext_dims":
        kw["ext_state"] = torch.empty((1, H, d, d // 2))
    elif case == "ws_small":
        kw["need"] = 65
    elif case == "ws_layout":
        kw["workspace"] = torch.empty((64, 2), dtype=torch.uint8)[:, 0]
    with pytest.raises((ValueError, TypeError)):
        la.check_scan_buffers(q, v, plan.info, **kw)


def test_allocation_follows_the_given_stream(monkeypatch):
    """With a stream argument the binding allocates inside that stream's
    context (so the caching allocator files the block under it)."""
    entered = []

    @contextlib.contextmanager
    def fake_stream(s):
        entered.append(s)
        yield

    monkeypatch.setattr(torch.cuda, "stream", fake_stream)
    marker = object()
    t = la._alloc((3, 4), torch.float32, "cpu", marker)
    assert entered == [marker] and t.shape == (3, 4)
    la._alloc((2,), torch.float32, "cpu", None)
    assert entered == [marker]


def test_pack_rejects_mismatched_request_arrays():
    """The library reads one branch count per request and sum(branch_count)
    branch lengths: shorter arrays would be read past their end, longer ones
    silently cut, so the binding refuses both."""
    la.pack([100, 50], [1, 2], [10, 20, 30])
    with pytest.raises(ValueError):
        la.pack([100, 50], [1, 2], [10, 20])
    with pytest.raises(ValueError):
        la.pack([100, 50], [1, 2], [10, 20, 30, 40])
    with pytest.raises(ValueError):
        la.pack([100, 50], [1], [10])


def test_build_refuses_kernels_with_scratch():
    """The build reads the compiler's resource remarks and names every kernel
    that needs scratch memory (the kernels are designed without)."""
    from chunked_linear_attention_packed_amd import build as b
    remarks = ("x.hip:1:1: remark: Function Name: k_ok [-Rpass-analysis=kernel-resource-usage]\n"
               "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n"
               "x.hip:9:1: remark: Function Name: k_spill [-Rpass-analysis=kernel-resource-usage]\n"
               "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 52 [-Rpass-analysis=kernel-resource-usage]\n")
    assert b._scratch_kernels(remarks) == [("k_spill", 52)]
    assert b._scratch_kernels(remarks.replace("52", "0")) == []
