"""Seeded synthetic inputs for the packed linear-attention scan.

Shared by the tests, the smoke check and the benchmark, for both the HIP path
and the CPU oracle.  This module draws random numbers and builds input arrays;
it holds none of the scan's arithmetic.

Workload shapes follow the page "Serving 0.88M TPS from Two RTXs and Mac
Minis": views of 500 to 18,000 tokens with 1 to hundreds of branches (section
"Batching in the Router", "Cost Model"), 8 behaviours per request (section
"Kernels"), a four-request pass and a 7,400-token pass (section "Kernels"),
hundreds of behaviours against one view (section "Long Requests").  The page
measured on private spans; these synthetic passes stand in for them.

Draw protocol (fixed): numpy.random.default_rng(seed); draw, in this order,
view lengths, branch counts, branch lengths (request order), then q, k, v as
float32 standard normals of shape [T, H, d] in that order.  k is multiplied by
1/sqrt(d) in float32, then every tensor is cast to the workload dtype with
round-to-nearest-even (torch's cast).  "Uniform a-b" is an inclusive integer
draw; "log-uniform a-b" is round(exp(U(ln a, ln b))) clipped to [a, b].
"""
import math
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "shapes", "draw_qkv",
           "ternary_qkv", "probe_qkv"]


@dataclass
class Workload:
    name: str
    seed: int
    H: int
    d: int
    dtype: str                       # "f32" or "bf16"
    view_len: np.ndarray = field(repr=False)
    branch_count: np.ndarray = field(repr=False)
    branch_len: np.ndarray = field(repr=False)
    q: object = field(default=None, repr=False)   # torch CPU tensors
    k: object = field(default=None, repr=False)
    v: object = field(default=None, repr=False)

    @property
    def n_tokens(self):
        return int(self.view_len.sum() + self.branch_len.sum())


def _fixed(n, x):
    return np.full(n, x, dtype=np.int64)


def _shape_view500(rng):
    return _fixed(1, 500), _fixed(1, 4), _fixed(4, 32)


def _shape_view7400(rng):
    return _fixed(1, 7400), _fixed(1, 8), _fixed(8, 48)


def _shape_req4(rng):
    vl = rng.integers(500, 18000, size=4, endpoint=True)
    bc = _fixed(4, 8)
    bl = rng.integers(24, 96, size=int(bc.sum()), endpoint=True)
    return vl, bc, bl


def _shape_view18000(rng):
    vl = _fixed(1, 18000)
    bc = _fixed(1, 256)
    bl = rng.integers(32, 128, size=256, endpoint=True)
    return vl, bc, bl


def _shape_req32(rng):
    u = rng.uniform(math.log(500), math.log(18000), size=32)
    vl = np.clip(np.rint(np.exp(u)), 500, 18000).astype(np.int64)
    bc = rng.integers(1, 64, size=32, endpoint=True)
    bl = rng.integers(24, 128, size=int(bc.sum()), endpoint=True)
    return vl, bc, bl


# name -> (seed, H, d, dtype, shape drawer)
WORKLOADS = {
    # 1 view of 500 tokens + 4 branches of 32, H=2, d=64, fp32
    "view500_br4x32_h2_d64_f32": (1001, 2, 64, "f32", _shape_view500),
    # 1 view of 7,400 tokens + 8 branches of 48, H=16, d=64, bf16
    "view7400_br8x48_h16_d64_bf16": (1002, 16, 64, "bf16", _shape_view7400),
    # 4 requests: views U[500,18000], 8 branches each of U[24,96], H=16, d=64
    "req4_view500-18000_br8x24-96_h16_d64_bf16": (1003, 16, 64, "bf16", _shape_req4),
    # 1 view of 18,000 tokens + 256 branches of U[32,128], H=16, d=64
    "view18000_br256x32-128_h16_d64_bf16": (1004, 16, 64, "bf16", _shape_view18000),
    # 32 requests: views logU[500,18000], U[1,64] branches of U[24,128], H=32, d=128
    "req32_view500-18000_br1-64x24-128_h32_d128_bf16": (1005, 32, 128, "bf16", _shape_req32),
    # the fp32 case scaled up to the 7,400-token pass (fp32 MFMA vs split bf16)
    "view7400_br8x48_h16_d64_f32": (1006, 16, 64, "f32", _shape_view7400),
}


def shapes(name):
    """Request shapes only (no tensors): (view_len, branch_count, branch_len)."""
    seed, H, d, dtype, drawer = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    return drawer(rng)


def _torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def draw_qkv(rng, T, H, d, dtype, dv=None):
    """q, k, v as in the draw protocol; returns torch CPU tensors."""
    import torch
    dv = d if dv is None else dv
    td = _torch_dtype(dtype)
    out = []
    for name, last in (("q", d), ("k", d), ("v", dv)):
        x = rng.standard_normal((T, H, last), dtype=np.float32)
        if name == "k":
            x *= np.float32(1.0 / math.sqrt(d))
        out.append(torch.from_numpy(x).to(td))
        del x
    return tuple(out)


def workload(name, with_tensors=True):
    """Build a named workload with its canonical seeded inputs."""
    seed, H, d, dtype, drawer = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    vl, bc, bl = drawer(rng)
    w = Workload(name, seed, H, d, dtype, vl.astype(np.int64), bc.astype(np.int64),
                 bl.astype(np.int64))
    if with_tensors:
        w.q, w.k, w.v = draw_qkv(rng, w.n_tokens, H, d, dtype)
    return w


def ternary_qkv(seed, T, H, d, dtype, dv=None):
    """q, k, v with entries drawn uniformly from {-1, 0, 1}."""
    import torch
    dv = d if dv is None else dv
    rng = np.random.default_rng(seed)
    td = _torch_dtype(dtype)
    return tuple(torch.from_numpy(rng.integers(-1, 1, size=(T, H, last), endpoint=True)
                                  .astype(np.float32)).to(td)
                 for last in (d, d, dv))


def probe_qkv(seg_offsets, branch_parent, H, d, digit=0):
    """Inputs of the exact indexing probe: q = k = e_0 for every token and
    head, v of a token = one-hot of its segment's code.  Segment s gets code
    s; with digit > 0 the code's base-d digit of that order is used, so passes
    with more than d segments are covered by several probes.  fp32 only.
    """
    import torch
    seg_offsets = np.asarray(seg_offsets)
    T = int(seg_offsets[-1])
    q = np.zeros((T, H, d), dtype=np.float32)
    q[:, :, 0] = 1.0
    v = np.zeros((T, H, d), dtype=np.float32)
    for s in range(len(branch_parent)):
        code = (s // d ** digit) % d
        v[seg_offsets[s]:seg_offsets[s + 1], :, code] = 1.0
    t = torch.from_numpy
    return t(q), t(q.copy()), t(v)

