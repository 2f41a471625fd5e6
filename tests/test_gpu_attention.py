"""GPU parity of the tree-masked softmax attention (la_attn_packed) against
the fp64 oracle (oracle/attention.py), through the C ABI.

Tolerance: row-normalised max relative error 2e-2 (bf16 inputs), the same
rule as the scan.  Shard branches reading their view from external K/V arrays
are compared bit for bit with the same branches in the full pass."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import oracle_pool
import chunked_linear_attention_packed_amd as la

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2


def _run(q, k, v, so, bp, scale, ext_len=None, ext_k=None, ext_v=None):
    plan = la.attn_plan(so, bp, ext_len)
    ek = None if ext_k is None else ext_k.to(DEV).contiguous()
    ev = None if ext_v is None else ext_v.to(DEV).contiguous()
    out = la.attn_packed(q.to(DEV), k.to(DEV), v.to(DEV), plan, scale, ext_k=ek, ext_v=ev)
    torch.cuda.synchronize()
    return out.cpu()


STRUCTS = {
    "view1": ([1], [0], []),
    "view63": ([63], [0], []),
    "view64": ([64], [0], []),
    "view65": ([65], [0], []),
    "view200_br3": ([200], [3], [1, 64, 130]),
    "two_requests": ([129, 70], [2, 1], [65, 5, 64]),
    "branch_len1_view_len1": ([1, 3], [2, 1], [1, 1, 2]),
}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("name", list(STRUCTS))
def test_attention_matches_oracle(name, d):
    vl, bc, bl = STRUCTS[name]
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    H = 3
    q, k, v = synth.draw_qkv(np.random.default_rng(sum(name.encode()) + d), int(so[-1]),
                             H, d, "bf16")
    out = _run(q, k, v, so, bp, 1.0)
    ref = oracle.attention_dense(q, k, v, so, bp, 1.0)
    err = oracle.row_rel_err(out, ref)
    print(f"{name} d={d}: err {err:.2e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("scale", [0.05, 8.0])
def test_attention_extreme_scales(scale):
    """Near-uniform weights and near-argmax weights (large logits: the
    running maximum must keep exp() finite)."""
    so, bp, _ = oracle.pack_segments([300], [2], [40, 90])
    q, k, v = synth.draw_qkv(np.random.default_rng(3), int(so[-1]), 2, 64, "bf16")
    out = _run(q, k, v, so, bp, scale)
    assert torch.isfinite(out.float()).all()
    err = oracle.row_rel_err(out, oracle.attention_dense(q, k, v, so, bp, scale))
    print(f"scale {scale}: err {err:.2e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("d", [64, 128])
def test_shard_branches_from_external_view_kv(d):
    H = 2
    vl, bc, bl = [150], [4], [20, 64, 65, 3]
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    q, k, v = synth.draw_qkv(np.random.default_rng(21), int(so[-1]), H, d, "bf16")
    full = _run(q, k, v, so, bp, 1.0)
    # the branches alone, their view's K/V given as external view 0
    a = int(so[1])
    so_s = np.asarray(so[1:]) - a
    bp_s = np.full(len(bl), -2)
    shard = _run(q[a:], k[a:], v[a:], so_s, bp_s, 1.0, ext_len=[vl[0]], ext_k=k[:a],
                 ext_v=v[:a])
    assert torch.equal(shard, full[a:])
    ref = oracle.attention_dense(q[a:], k[a:], v[a:], so_s, bp_s, 1.0,
                                 ext_kv=[(k[:a], v[:a])])
    assert oracle.row_rel_err(shard, ref) <= TOL


def test_several_external_views_and_a_packed_view_in_one_pass():
    H, d = 2, 64
    rng = np.random.default_rng(22)
    ext_len = [70, 5, 200]
    ek, ev, _ = synth.draw_qkv(rng, sum(ext_len), H, d, "bf16")
    # segments: shard branch of ext view 2, a view, its branch, shard branch of ext view 0
    so = np.array([0, 30, 130, 200, 201])
    bp = np.array([-4, -1, 1, -2])
    q, k, v = synth.draw_qkv(rng, int(so[-1]), H, d, "bf16")
    out = _run(q, k, v, so, bp, 1.0, ext_len=ext_len, ext_k=ek, ext_v=ev)
    offs = np.concatenate([[0], np.cumsum(ext_len)])
    ext_kv = [(ek[offs[e]:offs[e + 1]], ev[offs[e]:offs[e + 1]]) for e in range(3)]
    ref = oracle.attention_dense(q, k, v, so, bp, 1.0, ext_kv=ext_kv)
    err = oracle.row_rel_err(out, ref)
    print(f"mixed external views: err {err:.2e}", flush=True)
    assert err <= TOL


def _attn_heads_worker(h):
    """fp64 attention oracle (attention_dense) for one head of the shared pass."""
    sh = oracle_pool.SHARED
    sl = slice(h, h + 1)
    return oracle.attention_dense(sh["q"][:, sl], sh["k"][:, sl], sh["v"][:, sl], sh["so"],
                                  sh["bp"], 1.0)


@pytest.mark.parametrize("name", ["view7400_br8x48_h16_d64_bf16",
                                  "view18000_br256x32-128_h16_d64_bf16"])
def test_attention_workload_full_parity(name):
    """The workload's whole pass compared element by element with the fp64
    attention oracle (every row of every head; heads on a process pool)."""
    w = synth.workload(name)
    so, bp, _ = oracle.pack_segments(w.view_len, w.branch_count, w.branch_len)
    plan = la.attn_plan(so, bp)
    out = la.attn_packed(w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), plan, 1.0)
    torch.cuda.synchronize()
    shared = dict(q=oracle_pool.to_f32(w.q), k=oracle_pool.to_f32(w.k),
                  v=oracle_pool.to_f32(w.v), so=so, bp=bp)
    parts = oracle_pool.run(_attn_heads_worker, list(range(w.H)), shared)
    ref = np.concatenate(parts, axis=1)
    err = oracle.row_rel_err(out.cpu(), ref)
    print(f"{name}: all {w.n_tokens} rows x {w.H} heads, err {err:.2e}", flush=True)
    assert err <= TOL


def test_attention_is_deterministic_and_overwrites_out():
    so, bp, _ = oracle.pack_segments([257], [2], [33, 70])
    q, k, v = (x.to(DEV) for x in synth.draw_qkv(np.random.default_rng(9), int(so[-1]), 4, 64,
                                                   "bf16"))
    plan = la.attn_plan(so, bp)
    a = la.attn_packed(q, k, v, plan, 1.0)
    b = torch.full_like(a, float("nan"))
    la.attn_packed(q, k, v, plan, 1.0, out=b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_attention_rejects_bad_arguments():
    so, bp, _ = oracle.pack_segments([10], [1], [5])
    plan = la.attn_plan(so, bp)
    q = torch.zeros((15, 2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(la.LinAttnError):
        la.attn_packed(q.float(), q.float(), q.float(), plan, 1.0)      # fp32: unsupported
    q96 = torch.zeros((15, 2, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(la.LinAttnError):
        la.attn_packed(q96, q96, q96, plan, 1.0)                         # d = 96
    with pytest.raises(ValueError):
        la.attn_packed(q[:10], q[:10], q[:10], plan, 1.0)                # token count
    for bad_scale in (0.0, -1.0, float("inf")):
        with pytest.raises(la.LinAttnError):
            la.attn_packed(q, q, q, plan, bad_scale)                     # scale must be > 0
    ext_plan = la.attn_plan([0, 4], [-2], ext_len=[7])
    q4 = torch.zeros((4, 2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        la.attn_packed(q4, q4, q4, ext_plan, 1.0)                        # ext arrays missing


def test_hand_worked_example_on_the_gpu():
    """tests/golden/attention_hand_example.json, zero-padded to d = 64 (the
    padding changes no dot product): every weight is a power of two and every
    v an integer, so only the final bf16 rounding (and the fp32 reciprocal of
    the sum) separates the kernel from the exact values."""
    with open(os.path.join(os.path.dirname(__file__), "golden",
                           "attention_hand_example.json")) as f:
        g = json.load(f)
    T = len(g["out"])
    pad = lambda key: torch.nn.functional.pad(torch.tensor(g[key], dtype=torch.float32),
                                              (0, 64 - len(g[key][0])))
    q, k, v = (pad(x).reshape(T, 1, 64).to(torch.bfloat16) for x in ("q", "k", "v"))
    out = _run(q, k, v, g["seg_offsets"], g["branch_parent"], math.log(2.0))
    exp = torch.tensor(g["out"], dtype=torch.float64)[:, 0]
    got = out[:, 0, 0].double()
    assert torch.all((got - exp).abs() <= exp.abs() * 2.0 ** -8 + 1e-6), (got, exp)
    assert torch.all(out[:, 0, 1:] == 0)



@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("first_half_high", [True, False])
def test_attention_key_halves_far_apart(d, first_half_high):
    """Keys whose scores differ by about 24 between the first and the second
    32 positions of every 64-key block: each query's two key halves (kept
    apart until the end of the walk) have maxima far apart, so combining them
    rescales one side to almost nothing -- the first half or the second."""
    H = 2
    so, bp, _ = oracle.pack_segments([300], [2], [40, 90])
    T = int(so[-1])
    rng = np.random.default_rng(47 + d + int(first_half_high))
    qn = rng.standard_normal((T, H, d)).astype(np.float32) * 0.1 + 1.0
    pos = np.arange(T) - np.repeat(so[:-1], np.diff(so))   # position in its segment
    sign = np.where((pos % 64) < 32, 1.0, -1.0).astype(np.float32)
    if not first_half_high:
        sign = -sign
    kn = rng.standard_normal((T, H, d)).astype(np.float32) * 0.05 + \
        sign[:, None, None] * (12.0 / d)
    vn = rng.standard_normal((T, H, d)).astype(np.float32)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16) for x in (qn, kn, vn))
    out = _run(q, k, v, so, bp, 1.0)
    ref = oracle.attention_dense(q, k, v, so, bp, 1.0)
    err = oracle.row_rel_err(out, ref)
    print(f"key halves apart d={d} first_high={first_half_high}: err {err:.2e}", flush=True)
    assert torch.isfinite(out.float()).all()
    assert err <= TOL

@pytest.mark.parametrize("d", [64, 128])
def test_attention_rising_scores_rescale_every_block(d):
    """Scores that grow along the keys, so that nearly every key block raises
    a query's running maximum by far more than the lazy-rescale slack: the
    rescale path runs block after block and must still give the softmax."""
    H = 2
    so, bp, _ = oracle.pack_segments([520], [2], [70, 130])
    T = int(so[-1])
    rng = np.random.default_rng(31)
    qn = rng.standard_normal((T, H, d)).astype(np.float32) * 0.1 + 1.0
    ramp = np.linspace(0.0, 1.0, T, dtype=np.float32)[:, None, None]
    kn = rng.standard_normal((T, H, d)).astype(np.float32) * 0.05 + ramp * (20.0 / d)
    vn = rng.standard_normal((T, H, d)).astype(np.float32)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16) for x in (qn, kn, vn))
    out = _run(q, k, v, so, bp, 1.0)
    ref = oracle.attention_dense(q, k, v, so, bp, 1.0)
    err = oracle.row_rel_err(out, ref)
    print(f"rising scores d={d}: err {err:.2e}", flush=True)
    assert torch.isfinite(out.float()).all()
    assert err <= TOL
