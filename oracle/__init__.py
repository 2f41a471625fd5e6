"""CPU oracle for the packed chunked causal linear-attention scan.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import anything from this package. The
product path (the HIP library and its Python binding) never imports, calls or
links it, and this package never imports the product path.

Source: the page "Serving 0.88M TPS from Two RTXs and Mac Minis", sections
"The Workload" (one long view, many short branches; branches attend to the
view, not to each other), "Kernels" (linear attention in 64-token chunks; one
scan per pass; packed branch passes) and "Long Requests" (branch shards seeded
from a cached view state).

Everything here is plain numpy in float64. Inputs are the exact stored values
(bf16 or fp32) upcast to float64, so input rounding is not an error source.

Contents:
  pack.pack_segments     -- request shapes -> segment CSR (own packer)
  scan.scan_recurrence   -- THE oracle: token-by-token fp64 state recurrence
  scan.scan_bruteforce   -- O(T^2) tree-masked (QK^T)V; pins the recurrence
  scan.scan_chunked      -- chunked fp64 evaluator; pins chunk-size invariance
  scan.sample_rows       -- closed form for selected tokens (large passes)
  scan.view_states       -- final states of selected views (large passes)
  attention.attention_dense -- tree-masked softmax attention of a pass (the
                           other layer type, section "The Workload")
  attention.attention_rows  -- the same for selected tokens
  metrics.row_rel_err    -- row-normalised max relative error
"""
from .pack import pack_segments, view_ordinals
from .scan import scan_recurrence, scan_bruteforce, scan_chunked, sample_rows, view_states
from .attention import attention_dense, attention_rows, attention_flops
from .metrics import row_rel_err, state_rel_err

__all__ = ["pack_segments", "view_ordinals", "scan_recurrence", "scan_bruteforce",
           "scan_chunked", "sample_rows", "view_states", "attention_dense", "attention_rows",
           "attention_flops", "row_rel_err", "state_rel_err"]
