"""Entry points called from several host threads at once.

Each thread runs steps of its own batch on its own stream with its own
workspace; the batches are small enough to run as two stream groups, so
both threads also share the library's second stream, its fork and join
events, and its table-image cache.  The results must be bit-identical to the
same steps run one thread after the other on the current stream.
"""
import threading

import pytest
import torch

import dmuon_inputs as di
from tests.gpu_helpers import DEV, upload

pytestmark = pytest.mark.gpu

SHAPES = {0: [(1024, 1024)] * 4, 1: [(1024, 2048), (2048, 1024), (1536, 1536), (1536, 1536)]}
STEPS = 6


def _state(tid):
    shapes = SHAPES[tid]
    ps = [upload(di.normal_matrix(r, c, 0.02, "bf16", 0, (70 + tid, i))[0], "bf16") for i, (r, c) in enumerate(shapes)]
    ms = [torch.zeros(r, c, dtype=torch.float32, device=DEV) for r, c in shapes]
    gs = [[upload(di.normal_matrix(r, c, 1e-3, "bf16", 0, (72 + tid, s, i))[0], "bf16")
           for i, (r, c) in enumerate(shapes)] for s in range(STEPS)]
    return ps, ms, gs


def test_threads_on_own_streams_match_sequential(lib):
    for tid in SHAPES:
        assert len(lib.dmuon_plan_describe(SHAPES[tid])["stream_groups"]) == 2, tid
    # sequential reference on the current stream
    ref = {}
    for tid in SHAPES:
        ps, ms, gs = _state(tid)
        for s in range(STEPS):
            lib.dmuon_step(ps, gs[s], ms)
        torch.cuda.synchronize()
        ref[tid] = (ps, ms)

    states = {tid: _state(tid) for tid in SHAPES}
    streams = {tid: torch.cuda.Stream() for tid in SHAPES}
    workspaces = {}
    for tid in SHAPES:
        ps, ms, gs = states[tid]
        workspaces[tid] = torch.empty(lib.dmuon_step_workspace_size(ps, gs[0], ms), dtype=torch.uint8, device=DEV)
        streams[tid].wait_stream(torch.cuda.current_stream())
    errors = []
    barrier = threading.Barrier(len(SHAPES))

    def run(tid):
        try:
            ps, ms, gs = states[tid]
            barrier.wait()
            for s in range(STEPS):
                lib.dmuon_step(ps, gs[s], ms, workspace=workspaces[tid], stream=streams[tid])
        except Exception as e:          # reported on the main thread
            errors.append((tid, repr(e)))

    threads = [threading.Thread(target=run, args=(tid,)) for tid in SHAPES]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads)
    torch.cuda.synchronize()
    assert not errors, errors
    for tid in SHAPES:
        ps, ms, _ = states[tid]
        rps, rms = ref[tid]
        for i in range(len(ps)):
            assert torch.equal(ps[i], rps[i]) and torch.equal(ms[i], rms[i]), (tid, i)
