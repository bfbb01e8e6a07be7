"""GPU parity of the whole step (dmuon_step) against the oracle, plus the
properties the step must keep: matrix independence, skipped matrices,
determinism and bit-identical resume.

Parity measures (relative Frobenius error):
  momentum buffer after every step        <= 1e-6
  parameter change W_new - W_old          <= 2e-2 (bf16 NS) / 1e-4 (fp32 NS)
"""
import time

import numpy as np
import pytest
import torch

import dmuon_inputs as di
from oracle import muon as orc
from tests.gpu_helpers import DEV, bf16_ulp, check_param_step, f64, rel, upload

pytestmark = pytest.mark.gpu

NS_TOL = {"bf16": 2e-2, "f32": 1e-4}


def _state(w: di.Workload, idx):
    params, exact = [], []
    for i in idx:
        raw, x = di.param_init(w, i)
        params.append(upload(raw, w.param_dtype))
        exact.append(x)
    moms = [torch.zeros(w.matrices[i].rows, w.matrices[i].cols, dtype=torch.float32, device=DEV) for i in idx]
    return params, exact, moms


def _grads(w, idx, step):
    out = [di.grad_at(w, i, step) for i in idx]
    return [upload(raw, w.grad_dtype) for raw, _ in out], [x for _, x in out]


def _hp(w, **over):
    hp = w.hparams()
    hp.update(over)
    return hp


@pytest.mark.parametrize("prec", ["bf16", "f32"])
@pytest.mark.parametrize("backend", ["gram", "direct"])
def test_step_small_workload(lib, prec, backend):
    """The single fp32 256 x 512 matrix, one step, both NS modes and forms."""
    w = di.workload(0)
    params, w0, moms = _state(w, [0])
    grads, g = _grads(w, [0], 0)
    lib.dmuon_step(params, grads, moms, **_hp(w, ns_precision=prec, ns_backend=backend))
    torch.cuda.synchronize()
    w_ref, m_ref, _, _ = orc.muon_step(w0[0], g[0], np.zeros_like(g[0]), lr=w.lr, momentum=w.momentum,
                                       nesterov=w.nesterov, ns_steps=w.ns_steps,
                                       weight_decay=w.weight_decay, ns_backend=backend,
                                       param_dtype=w.param_dtype)
    assert rel(f64(moms[0]), m_ref) <= 1e-6
    err = check_param_step(f64(params[0]), w0[0], w_ref, w.param_dtype, NS_TOL[prec], prec)
    print(f"256x512 {backend} {prec}: update rel err {err:.3e}")


# wide, tall, square, ragged tails and edges; the all-bf16 batch takes the
# path where the last product updates the parameter itself, the mixed one
# the separate update pass
RAGGED_SPECS = {
    "mixed": [(256, 512, "bf16"), (768, 256, "f32"), (1000, 1500, "bf16"), (384, 384, "f32"),
              (130, 70, "bf16"), (2048, 128, "bf16")],
    "bf16": [(256, 512, "bf16"), (1000, 1500, "bf16"), (1500, 1000, "bf16"), (130, 70, "bf16"),
             (70, 130, "bf16"), (2048, 128, "bf16"), (33, 1000, "bf16"), (1003, 37, "bf16"),
             (384, 384, "bf16")],
}


@pytest.mark.parametrize("batch", ["mixed", "bf16"])
@pytest.mark.parametrize("prec", ["bf16", "f32"])
def test_step_ragged_multi_step(lib, prec, gemm_tile, batch):
    """A batch of differently shaped matrices over three steps; the oracle
    runs its own trajectory (its own parameters and momenta, rounded to the
    parameter dtype each step) from the same start and gradients.  Checked
    after every step: the momentum (relative error <= 1e-6) and the change of
    each parameter since the start, within the NS tolerance plus the
    parameter roundings of both trajectories (one bf16 ulp per step)."""
    specs = RAGGED_SPECS[batch]
    rng = np.random.default_rng(11)
    params, w0, moms, m_ref, w_ref = [], [], [], [], []
    for i, (r, c, dt) in enumerate(specs):
        raw, x = di.normal_matrix(r, c, 0.02, dt, seed=0, tag=(20, i))
        params.append(upload(raw, dt))
        w0.append(x)
        w_ref.append(x.copy())
        moms.append(torch.zeros(r, c, dtype=torch.float32, device=DEV))
        m_ref.append(np.zeros((r, c)))
    hp = dict(lr=0.02, momentum=0.95, nesterov=True, ns_steps=5, weight_decay=0.1,
              ns_backend="gram", ns_precision=prec)
    for step in range(3):
        gs = [di.normal_matrix(r, c, 1e-3 * float(np.exp(rng.standard_normal())), dt, seed=0,
                               tag=(21, i, step)) for i, (r, c, dt) in enumerate(specs)]
        grads = [upload(raw, dt) for (raw, _), (_, _, dt) in zip(gs, specs)]
        lib.dmuon_step(params, grads, moms, **hp)
        torch.cuda.synchronize()
        for i, (r, c, dt) in enumerate(specs):
            w_ref[i], m_ref[i], _, _ = orc.muon_step(w_ref[i], gs[i][1], m_ref[i], ns_backend="gram",
                                                     weight_decay=0.1, param_dtype=dt)
            assert rel(f64(moms[i]), m_ref[i]) <= 1e-6, (step, i)
            got = f64(params[i])
            d_ref = w_ref[i] - w0[i]
            err = rel(got - w0[i], d_ref)
            allow = 0.0
            if dt == "bf16":
                allow = (step + 1) * float(np.linalg.norm(bf16_ulp(got)) / np.linalg.norm(d_ref))
            assert err <= NS_TOL[prec] + allow, (step, i, (r, c), err, allow)
            assert np.isfinite(got).all()
            print(f"step {step} {r}x{c} {dt} ns={prec} tile={gemm_tile}: change rel err {err:.3e} "
                  f"(rounding allowance {allow:.1e})")


def test_step_nan_isolation_and_skip(lib):
    """A non-finite gradient poisons only its own matrix; a NULL gradient
    leaves its matrix (param and momentum) untouched."""
    shapes = [(256, 512), (512, 256), (384, 384)]
    def fresh():
        ps = [upload(di.normal_matrix(r, c, 0.02, "bf16", 0, (30, i))[0], "bf16") for i, (r, c) in enumerate(shapes)]
        ms = [torch.full((r, c), 0.5, dtype=torch.float32, device=DEV) for r, c in shapes]
        gs = [upload(di.normal_matrix(r, c, 1e-3, "bf16", 0, (31, i))[0], "bf16") for i, (r, c) in enumerate(shapes)]
        return ps, ms, gs
    p1, m1, g1 = fresh()
    g1[0][3, 5] = float("nan")
    lib.dmuon_step(p1, g1, m1)
    p2, m2, g2 = fresh()
    lib.dmuon_step(p2[1:], g2[1:], m2[1:])
    torch.cuda.synchronize()
    assert torch.isnan(p1[0].float()).any()
    for i in (1, 2):
        assert torch.equal(p1[i], p2[i]) and torch.equal(m1[i], m2[i])
    p3, m3, g3 = fresh()
    before_p, before_m = p3[1].clone(), m3[1].clone()
    lib.dmuon_step(p3, [g3[0], None, g3[2]], m3)
    torch.cuda.synchronize()
    assert torch.equal(p3[1], before_p) and torch.equal(m3[1], before_m)
    assert torch.equal(p3[2], p2[2])


@pytest.mark.parametrize("prec", ["bf16", "f32"])
def test_step_deterministic_and_resume(lib, prec, gemm_tile):
    """Two runs are bit-identical, and a run stopped after step 2 and resumed
    from copies of (params, momenta) matches the uninterrupted run (every
    GEMM kernel: both precisions, both tile edges of each)."""
    w = di.workload(0)
    shapes = [(256, 512), (640, 256), (1024, 1024)]
    def init():
        ps = [upload(di.normal_matrix(r, c, 0.02, "bf16", 0, (40, i))[0], "bf16") for i, (r, c) in enumerate(shapes)]
        ms = [torch.zeros(r, c, dtype=torch.float32, device=DEV) for r, c in shapes]
        return ps, ms
    grads = [[upload(di.normal_matrix(r, c, 1e-3, "bf16", 0, (41, i, s))[0], "bf16")
              for i, (r, c) in enumerate(shapes)] for s in range(4)]
    pa, ma = init()
    pb, mb = init()
    for s in range(4):
        lib.dmuon_step(pa, grads[s], ma, ns_precision=prec)
        lib.dmuon_step(pb, grads[s], mb, ns_precision=prec)
    pc, mc = init()
    for s in range(2):
        lib.dmuon_step(pc, grads[s], mc, ns_precision=prec)
    torch.cuda.synchronize()
    saved_p = [p.cpu().clone() for p in pc]
    saved_m = [m.cpu().clone() for m in mc]
    pd = [p.to(DEV) for p in saved_p]
    md = [m.to(DEV) for m in saved_m]
    for s in range(2, 4):
        lib.dmuon_step(pd, grads[s], md, ns_precision=prec)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(pa[i], pb[i]) and torch.equal(ma[i], mb[i])
        assert torch.equal(pa[i], pd[i]) and torch.equal(ma[i], md[i])


def test_step_decoder_layer_full_size(lib):
    """The 3B decoder layer's seven projections at full size: one step checked
    in full against the oracle; momentum checked over ten steps."""
    w = di.workload(1)
    idx = list(range(len(w.matrices)))
    params, w0, moms = _state(w, idx)
    m_ref = [np.zeros((m.rows, m.cols)) for m in w.matrices]
    for step in range(w.steps):
        grads, g = _grads(w, idx, step)
        lib.dmuon_step(params, grads, moms, **w.hparams())
        torch.cuda.synchronize()
        for i in idx:
            m_ref[i], _ = orc.momentum_update(m_ref[i], g[i], w.momentum, w.nesterov)
            assert rel(f64(moms[i]), m_ref[i]) <= 1e-6, (step, i)
        if step == 0:
            t0 = time.time()
            for i in idx:
                w_ref, _, _, _ = orc.muon_step(w0[i], g[i], np.zeros_like(g[i]),
                                               ns_backend="gram", param_dtype="f32")
                err = check_param_step(f64(params[i]), w0[i], w_ref, "bf16", NS_TOL["bf16"],
                                       "bf16", what=w.matrices[i].name)
                print(f"{w.matrices[i].name} {w.matrices[i].rows}x{w.matrices[i].cols}: "
                      f"update rel err {err:.3e}", flush=True)
            print(f"oracle time {time.time() - t0:.1f}s", flush=True)
