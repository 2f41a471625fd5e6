"""The oracle's own packer: request shapes -> segment CSR.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Serving 0.88M TPS from Two RTXs and Mac Minis", section "The
Workload" (a request is one long view plus several short branches, branches
attend to their view but never to each other) and section "Kernels",
paragraph "Shared branch passes" (the branches of all requests of a pass go
through one packed forward). Section "Long Requests" adds branch shards that
carry the full view as a cached state instead of its tokens.

Packing order (a reading; the page fixes no order): request by request, the
view segment first, then that request's branches in the given order.

A request whose view length is 0 is a shard request: its view was scored in
an earlier pass and only the view's final state is supplied.  Its branches
take their initial state from external state row e, where e counts shard
requests in request order; they are marked with parent -2 - e.
"""
import numpy as np


def pack_segments(view_len, branch_count, branch_len):
    """Pack request shapes into segments.

    Returns (seg_offsets[n_seg+1], branch_parent[n_seg], view_ordinal[n_seg]),
    int64 arrays:
      seg_offsets    token offset of each segment in the packed pass
      branch_parent  -1 for a view; the segment index of its view for a
                     branch; -2 - e for a branch seeded from external state e
      view_ordinal   row of the final-state array for a view, -1 otherwise
    Raises ValueError for shapes the scan does not accept.
    """
    view_len = [int(x) for x in view_len]
    branch_count = [int(x) for x in branch_count]
    branch_len = [int(x) for x in branch_len]
    if len(view_len) != len(branch_count):
        raise ValueError("view_len and branch_count differ in length")
    if sum(branch_count) != len(branch_len):
        raise ValueError("branch_len does not hold sum(branch_count) entries")
    offsets = [0]
    parent = []
    ordinal = []
    n_views = 0
    n_ext = 0
    b = 0
    for r in range(len(view_len)):
        if view_len[r] < 0 or branch_count[r] < 0:
            raise ValueError("negative length or count")
        if view_len[r] == 0 and branch_count[r] == 0:
            raise ValueError("empty request")
        if view_len[r] > 0:
            my_view = len(parent)
            parent.append(-1)
            ordinal.append(n_views)
            n_views += 1
            offsets.append(offsets[-1] + view_len[r])
            seed = my_view
        else:
            seed = -2 - n_ext
            n_ext += 1
        for _ in range(branch_count[r]):
            if branch_len[b] < 1:
                raise ValueError("branch of length < 1")
            parent.append(seed)
            ordinal.append(-1)
            offsets.append(offsets[-1] + branch_len[b])
            b += 1
    if offsets[-1] >= 2**31:
        raise ValueError("pass too long for int32 token offsets")
    return (np.asarray(offsets, dtype=np.int64), np.asarray(parent, dtype=np.int64),
            np.asarray(ordinal, dtype=np.int64))


def view_ordinals(branch_parent):
    """Rank of each view segment among views (-1 for branches)."""
    out = np.full(len(branch_parent), -1, dtype=np.int64)
    n = 0
    for s, p in enumerate(branch_parent):
        if p == -1:
            out[s] = n
            n += 1
    return out
