"""dmuon_clip_grad_norm_noalloc inside a HIP graph.

The allocation-free clip passes its launch table as kernel arguments and
keeps its scratch in the library's device array, so a captured call replays
correctly.  The call is captured once (through torch's stream capture) and
the graph is replayed several times; before each replay the gradients are
reset eagerly and other eager work (a workspace clip of other tensors, and
a full synchronisation) runs in between.  Every replay must equal the eager
call bit for bit: the clipped gradients and the per-bucket totals.
"""
import pytest
import torch

import dmuon_inputs as di
from tests.gpu_helpers import DEV, upload

pytestmark = pytest.mark.gpu

# (rows, cols, dtype, std, bucket): sizes below, at and past one 64 KB chunk
SPECS = [(33, 65, "bf16", 1e-2, 0), (256, 128, "f32", 3.0, 0), (512, 512, "bf16", 0.5, 1),
         (1000, 70, "f32", 1e-2, 1), (64, 1024, "bf16", 3.0, 1)]


def _grads(tag):
    return [upload(di.normal_matrix(r, c, std, dt, seed=0, tag=(tag, i))[0], dt)
            for i, (r, c, dt, std, _) in enumerate(SPECS)]


def test_noalloc_clip_replays_in_graph(lib):
    buckets = [b for *_, b in SPECS]
    base = _grads(90)
    max_norm = [0.5, 2.0]                         # both buckets clip

    eager = [g.clone() for g in base]
    tot_eager = torch.zeros(2, dtype=torch.float64, device=DEV)
    lib.dmuon_clip_grad_norm_noalloc(eager, max_norm, buckets=buckets, total_norm=tot_eager)
    torch.cuda.synchronize()

    work = [g.clone() for g in base]
    tot = torch.zeros(2, dtype=torch.float64, device=DEV)
    # warm-up on a side stream (the library looks up its scratch address on
    # its first call on a device), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lib.dmuon_clip_grad_norm_noalloc(work, max_norm, buckets=buckets, total_norm=tot)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lib.dmuon_clip_grad_norm_noalloc(work, max_norm, buckets=buckets, total_norm=tot)

    others = _grads(91)
    for rep in range(3):
        for w, b in zip(work, base):
            w.copy_(b)
        tot.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (w, e) in enumerate(zip(work, eager)):
            assert torch.equal(w.view(torch.int16) if w.dtype == torch.bfloat16 else w.view(torch.int32),
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e.view(torch.int32)), (rep, i)
        assert torch.equal(tot, tot_eager), (rep, tot, tot_eager)
        # eager work between replays: a workspace clip of other tensors
        lib.dmuon_clip_grad_norm(others, 1.0)
        torch.cuda.synchronize()
