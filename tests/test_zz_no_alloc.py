"""The allocation-free clip, dmuon_clip_grad_norm_noalloc, against
dmuon_clip_grad_norm (the entry point with a caller workspace) on the same
inputs: bit-identical gradients and identical per-bucket totals, over two
calls in a row on one GPU, the second with a smaller input (fewer and
smaller gradients, fewer buckets) so that it runs on the scratch the first
call left behind.  Both calls go through the C ABI (the binding only
marshals arguments)."""
import math

import pytest
import torch

import dmuon_inputs as di
from tests.gpu_helpers import DEV, upload

pytestmark = pytest.mark.gpu

# (numel, dtype, bucket, scale, element offset into a larger buffer: the
# scalar path for unaligned gradients); sizes below, at and past the 64 KB
# block chunk (32768 bf16 / 16384 fp32 values)
FIRST = [(1000, "bf16", 0, 1e-2, 0), (32768, "bf16", 0, 3.0, 0), (32769, "f32", 1, 0.5, 0),
         (16384, "f32", 1, 2.0, 3), (250001, "bf16", 2, 1e-3, 1), (5, "f32", 2, 7.0, 0),
         (70000, "bf16", 3, 0.1, 0), (123457, "f32", 3, 1e-4, 0)]
SECOND = [(999, "f32", 0, 0.3, 0), (40000, "bf16", 1, 2.0, 5), (17, "bf16", 1, 1.0, 0)]


def _grads(specs, seed):
    out = []
    for i, (numel, dt, bucket, scale, off) in enumerate(specs):
        raw, _ = di.normal_matrix(1, numel + off, scale, dt, seed=seed, tag=(60, i))
        buf = upload(raw, dt)
        out.append(buf.view(-1)[off:off + numel])
    return out


@pytest.mark.parametrize("norm_type", [2.0, math.inf, 1.0])
def test_noalloc_clip_matches_workspace_clip(lib, norm_type):
    for call, specs in enumerate((FIRST, SECOND)):
        buckets = [b for _, _, b, _, _ in specs]
        nb = max(buckets) + 1
        ga = _grads(specs, seed=call)
        gb = [g.clone() for g in ga]
        # the norms of each bucket, so that max_norm clips some buckets and not others
        norms = []
        for b in range(nb):
            v = [g.double() for g, bb in zip(ga, buckets) if bb == b]
            if norm_type == math.inf:
                norms.append(max(float(x.abs().max()) for x in v))
            else:
                norms.append(float(sum(float((x.abs() ** norm_type).sum()) for x in v)) ** (1.0 / norm_type))
        max_norm = [norms[b] * (0.5 if b % 2 == 0 else 2.0) for b in range(nb)]
        ta = lib.dmuon_clip_grad_norm(ga, max_norm, norm_type=norm_type, buckets=buckets)
        tb = torch.full((nb,), -1.0, dtype=torch.float64, device=DEV)
        got = lib.dmuon_clip_grad_norm_noalloc(gb, max_norm, norm_type=norm_type, buckets=buckets, total_norm=tb)
        torch.cuda.synchronize()
        assert got is tb
        assert torch.equal(ta, tb), (call, ta.tolist(), tb.tolist())
        for i, (a, b) in enumerate(zip(ga, gb)):
            assert torch.equal(a, b), (call, i)
        for b in range(nb):
            assert abs(float(tb[b]) - norms[b]) <= 1e-9 * norms[b], (call, b)
        print(f"call {call} p={norm_type}: {len(specs)} gradients, {nb} buckets, totals {tb.tolist()}")
