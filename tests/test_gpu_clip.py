"""GPU parity of gradient clipping (dmuon_clip_grad_norm) against the oracle.

Tolerances: per-bucket totals relative 1e-12 (fp64 accumulation on both
sides, in different orders; general p goes through pow).  Both sides form
the clipped value as one fp64 product rounded once to the gradient's dtype,
so values are equal unless the two coefficients (each from its own total)
differ in their last bits and a product sits on a rounding boundary: every
value within one ulp of the oracle's and at least 99.99 % equal.  Buckets
with coefficient 1 stay bit-identical (not written).
"""
import math

import numpy as np
import pytest
import torch

import dmuon_inputs as di
from oracle import clip as orc_clip
from tests.gpu_helpers import DEV, assert_bf16_close, f64, upload

pytestmark = pytest.mark.gpu

# bf16 at even, f32 at odd positions; a block takes 64 KB of one gradient:
# whole chunks, one chunk plus a few elements, and sizes below one chunk
SIZES = [(1000,), (33, 7), (16384,), (16385,), (3, 70000), (8192 + 3,), (5,), (130, 257),
         (32768,), (16384,), (32769,)]


def _grads(seed, dtypes, scales):
    out = []
    for i, shape in enumerate(SIZES):
        dt = dtypes[i % len(dtypes)]
        raw, exact = di.normal_matrix(int(np.prod(shape)), 1, scales[i % len(scales)], dt, seed=seed, tag=(60, i))
        out.append((upload(raw.reshape(shape), dt), exact.reshape(shape), dt))
    return out


def _check_values(got, ref_unrounded, dt, what):
    ref = orc_clip.store(ref_unrounded, dt)
    if dt == "bf16":
        assert_bf16_close(got, ref, min_exact=0.9999, what=what)
    else:
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= ulp), what
        assert np.mean(got == ref) >= 0.9999, (what, float(np.mean(got == ref)))


@pytest.mark.parametrize("p", [2.0, 1.0, math.inf, 3.0])
def test_clip_buckets_parity(lib, p):
    gs = _grads(1, ["bf16", "f32"], [1e-2, 3.0, 0.5])
    buckets = [i % 3 for i in range(len(gs))]
    exact = [e for _, e, _ in gs]
    totals_ref = [orc_clip.grad_norm([e for e, b in zip(exact, buckets) if b == k], p) for k in range(3)]
    # bucket 0 and 1 clip, bucket 2 does not
    max_norm = [0.5 * totals_ref[0], 0.1 * totals_ref[1], 2.0 * totals_ref[2]]
    before = [t.clone() for t, _, _ in gs]
    totals = lib.dmuon_clip_grad_norm([t for t, _, _ in gs], max_norm, norm_type=p, buckets=buckets)
    torch.cuda.synchronize()
    out_ref, tot_ref, coef_ref = orc_clip.clip_grad_norm(exact, buckets, max_norm, p)
    tg = totals.cpu().numpy()
    for k in range(3):
        assert abs(tg[k] - tot_ref[k]) <= 1e-12 * tot_ref[k], (k, tg[k], tot_ref[k])
    assert coef_ref[2] == 1.0
    for i, (t, _, dt) in enumerate(gs):
        if buckets[i] == 2:
            assert torch.equal(t, before[i]), i
        else:
            _check_values(f64(t), out_ref[i], dt, f"grad {i} {SIZES[i]} {dt} p={p}")


def test_clip_misaligned_views_and_nan_isolation(lib):
    # gradients that start at odd element offsets (not 16-byte aligned)
    store = torch.zeros(3 * 40000 + 7, dtype=torch.bfloat16, device=DEV)
    views = [store[1:40001], store[40003:80003], store[80005:120005]]
    rng = np.random.default_rng(7)
    vals = []
    for v in views:
        raw, ex = di.to_storage(rng.standard_normal(v.numel()) * 2.0, "bf16")
        v.copy_(upload(raw, "bf16"))
        vals.append(ex)
    nan_grad = torch.full((1000,), 1.0, dtype=torch.float32, device=DEV)
    nan_grad[17] = float("nan")
    other = torch.full((1000,), 3.0, dtype=torch.float32, device=DEV)
    totals = lib.dmuon_clip_grad_norm(views + [nan_grad, other], [1.0, 1.0, 1.0],
                                      buckets=[0, 0, 0, 1, 2])
    torch.cuda.synchronize()
    out_ref, tot_ref, _ = orc_clip.clip_grad_norm(vals, [0, 0, 0], [1.0], 2.0)
    tg = totals.cpu().numpy()
    assert abs(tg[0] - tot_ref[0]) <= 1e-12 * tot_ref[0]
    for v, r in zip(views, out_ref):
        _check_values(f64(v), r, "bf16", "misaligned view")
    assert store[0].item() == 0.0 and store[40001].item() == 0.0 and store[-1].item() == 0.0
    assert math.isnan(tg[1]) and torch.isnan(nan_grad).all()
    ref2, t2, _ = orc_clip.clip_grad_norm([np.full(1000, 3.0)], [0], [1.0], 2.0)
    assert abs(tg[2] - t2[0]) <= 1e-12 * t2[0]
    _check_values(f64(other), ref2[0], "f32", "bucket next to a NaN")


def test_clip_deterministic(lib):
    gs = _grads(3, ["bf16"], [1.0])
    a = [t.clone() for t, _, _ in gs]
    b = [t.clone() for t, _, _ in gs]
    ta = lib.dmuon_clip_grad_norm(a, 1.0)
    tb = lib.dmuon_clip_grad_norm(b, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(ta, tb)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_clip_full_3b_stack(lib):
    """Every gradient of the 196-matrix stack (2.82 G bf16 values) in one
    bucket, clipping active.  The oracle cannot sum 2.82 G values in seconds,
    so the total is checked against the definition evaluated with float64
    device reductions, matrix by matrix; two sampled matrices go through the
    oracle (their own norms, then every element after clipping), and every
    matrix's norm must shrink by the coefficient."""
    w = di.workload(2)
    grads = []
    for i, m in enumerate(w.matrices):
        g = torch.empty(m.rows, m.cols, dtype=torch.bfloat16, device=DEV)
        di.torch_normal_(g, w.grad_std, seed=20000 + i)
        grads.append(g)
    sq = [float(g.double().square().sum()) for g in grads]
    total_ref = math.sqrt(math.fsum(sq))
    sample = [0, 4]
    before = {i: f64(grads[i]) for i in sample}
    for i in sample:
        assert math.isclose(orc_clip.grad_norm([before[i]], 2.0), math.sqrt(sq[i]), rel_tol=1e-12)
    max_norm = 0.25 * total_ref
    totals = lib.dmuon_clip_grad_norm(grads, max_norm)
    torch.cuda.synchronize()
    tg = float(totals.cpu()[0])
    assert abs(tg - total_ref) <= 1e-12 * total_ref, (tg, total_ref)
    coef = orc_clip.clip_coefficient(total_ref, max_norm)
    for i, g in enumerate(grads):
        r = math.sqrt(float(g.double().square().sum()) / sq[i])
        assert abs(r - coef) <= 1e-3 * coef, (i, r, coef)      # bf16 rounding of every element
    for i in sample:
        _check_values(f64(grads[i]), before[i] * coef, "bf16", f"matrix {i}")


@pytest.mark.parametrize("gdt", ["bf16", "f32"])
def test_clip_fused_into_step_is_bitwise_equal(lib, gdt):
    """dmuon_clip_coefficients + dmuon_step with grad_scale gives the same
    parameters and momenta, bit for bit, as dmuon_clip_grad_norm (in place)
    + dmuon_step, and leaves the gradients untouched; two clipped buckets, a
    bucket that does not clip and a matrix left unscaled (index -1, in a
    bucket whose coefficient is 1)."""
    shapes = [(256, 512), (1000, 1500), (130, 70), (2048, 128), (384, 384), (70, 130)]
    buckets = [0, 0, 1, 1, 2, 2]
    pdt = "bf16"
    params_a, params_b, moms_a, moms_b, grads = [], [], [], [], []
    for i, (r, c) in enumerate(shapes):
        raw, _ = di.normal_matrix(r, c, 0.02, pdt, seed=0, tag=(90, i))
        params_a.append(upload(raw, pdt))
        params_b.append(upload(raw, pdt))
        graw, _ = di.normal_matrix(r, c, 1e-2 * (i + 1), gdt, seed=0, tag=(91, i))
        grads.append(upload(graw, gdt))
        moms_a.append(torch.zeros(r, c, dtype=torch.float32, device=DEV))
        moms_b.append(torch.zeros(r, c, dtype=torch.float32, device=DEV))
    totals = lib.dmuon_clip_grad_norm([g.clone() for g in grads], [1e30] * 3, buckets=buckets)
    torch.cuda.synchronize()
    t = totals.cpu().numpy()
    max_norm = [0.3 * t[0], 0.5 * t[1], 2.0 * t[2]]
    grads_a = [g.clone() for g in grads]
    grads_b = [g.clone() for g in grads]
    ta = lib.dmuon_clip_grad_norm(grads_a, max_norm, buckets=buckets)
    lib.dmuon_step(params_a, grads_a, moms_a)
    tb = torch.empty(3, dtype=torch.float64, device=DEV)
    coefs = lib.dmuon_clip_coefficients(grads_b, max_norm, buckets=buckets, total_norm=tb)
    index = list(buckets)
    index[5] = -1
    lib.dmuon_step(params_b, grads_b, moms_b, grad_scale=coefs, grad_scale_index=index)
    torch.cuda.synchronize()
    c = coefs.cpu().numpy()
    assert c[0] < 1.0 and c[1] < 1.0 and c[2] == 1.0
    assert torch.equal(ta, tb)
    for i in range(len(shapes)):
        assert torch.equal(grads_b[i], grads[i]), i
        assert torch.equal(moms_a[i], moms_b[i]), i
        assert torch.equal(params_a[i], params_b[i]), i
