"""GPU parity of each stage of the step against the oracle, through the C ABI.

Tolerances (relative Frobenius error unless stated):
  momentum buffer and fp32 NS input  <= 1e-6
  NS output, bf16 products           <= 2e-2
  NS output, fp32 products           <= 1e-4
  update, fp32 parameters            <= 1e-6
  update, bf16 parameters            every element within one bf16 ulp of the
                                     oracle's rounded value (plus the fp32
                                     evaluation error of w*(1-lr*wd) and the
                                     fused multiply-add), >= 99.9 % equal
"""
import numpy as np
import pytest
import torch

import dmuon_inputs as di
from oracle import muon as orc
from tests.gpu_helpers import DEV, assert_bf16_close, f64, rel, upload

pytestmark = pytest.mark.gpu

NS_TOL = {"bf16": 2e-2, "f32": 1e-4}

# several tiles and ragged tails in both orientations
SHAPES = [(256, 512), (512, 256), (1000, 1500), (1500, 1000), (130, 70), (128, 2048),
          (2048, 128), (384, 384), (200, 700), (64, 64), (1, 300)]


def _normal(rows, cols, std, dtype, tag):
    return di.normal_matrix(rows, cols, std, dtype, seed=0, tag=tag)


@pytest.mark.parametrize("nesterov", [True, False])
@pytest.mark.parametrize("gdt,udt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_momentum_stage(lib, nesterov, gdt, udt):
    shapes = [(256, 512), (512, 256), (1000, 1500), (130, 70), (33, 5)]
    mus = 0.95
    moms = [torch.zeros(r, c, dtype=torch.float32, device=DEV) for r, c in shapes]
    m_ref = [np.zeros((r, c)) for r, c in shapes]
    tdt = torch.float32 if udt == "f32" else torch.bfloat16
    for step in range(3):
        grads_raw = [_normal(r, c, 1e-3, gdt, (1, i, step)) for i, (r, c) in enumerate(shapes)]
        grads = [upload(raw, gdt) for raw, _ in grads_raw]
        outs = [torch.full((min(r, c), max(r, c)), float("nan"), dtype=tdt, device=DEV) for r, c in shapes]
        sumsq = torch.zeros(len(shapes), dtype=torch.float64, device=DEV)
        lib.dmuon_momentum(grads, moms, outs, sumsq, momentum=mus, nesterov=nesterov)
        torch.cuda.synchronize()
        for i, (r, c) in enumerate(shapes):
            m_ref[i], u = orc.momentum_update(m_ref[i], grads_raw[i][1], mus, nesterov)
            assert rel(f64(moms[i]), m_ref[i]) <= 1e-6, (step, i)
            u_wide = u.T if r > c else u
            got = f64(outs[i])
            if udt == "f32":
                assert rel(got, u_wide) <= 1e-6, (step, i)
            else:
                assert_bf16_close(got, orc.round_to_bf16(u_wide), what=f"U {step} {i}")
            ss = float(sumsq[i].item())
            assert abs(ss - float(np.sum(u * u))) <= 1e-6 * float(np.sum(u * u)), (step, i)


@pytest.mark.parametrize("pdt,odt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_update_stage(lib, pdt, odt, wd):
    shapes = [(256, 512), (512, 256), (1000, 1500), (130, 70), (7, 3)]
    lr = 0.02
    params, refs, slack = [], [], []
    updates = []
    for i, (r, c) in enumerate(shapes):
        w_raw, w = _normal(r, c, 0.02, pdt, (2, i))
        o_raw, o = _normal(r, c, 1.0 / np.sqrt(max(r, c)), odt, (3, i))
        params.append(upload(w_raw, pdt))
        updates.append(upload(o_raw, odt))
        ref = orc.apply_update(w, o, lr, wd)
        refs.append(orc.round_to_bf16(ref) if pdt == "bf16" else ref)
        # the kernel evaluates w*(1-lr*wd) and the fused multiply-add in fp32
        slack.append(4 * 2.0 ** -24 * (np.abs(w) + orc.lr_scale(r, c) * lr * np.abs(o)))
    lib.dmuon_apply_update(params, updates, lr=lr, weight_decay=wd)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        got = f64(params[i])
        if pdt == "f32":
            assert rel(got, refs[i]) <= 1e-6, i
        else:
            assert_bf16_close(got, refs[i], what=f"W {i}", slack=slack[i])


@pytest.mark.parametrize("prec", ["bf16", "f32"])
@pytest.mark.parametrize("backend", ["gram", "direct"])
def test_orthogonalize(lib, prec, backend, gemm_tile):
    inputs, refs = [], []
    for i, (r, c) in enumerate(SHAPES):
        raw, x = _normal(r, c, 1e-2, "f32", (4, i))
        inputs.append(upload(raw, "f32"))
        refs.append(orc.orthogonalize(x, 5, backend, None, 1e-7))
    outs = [torch.empty_like(t) for t in inputs]
    lib.dmuon_orthogonalize(inputs, outs, ns_backend=backend, ns_precision=prec)
    torch.cuda.synchronize()
    for i, shape in enumerate(SHAPES):
        err = rel(f64(outs[i]), refs[i])
        print(f"{shape} {backend} {prec} tile={gemm_tile}: NS rel err {err:.3e}")
        assert err <= NS_TOL[prec], (shape, err)


@pytest.mark.parametrize("prec", ["bf16", "f32"])
def test_orthogonalize_bf16_io_inplace(lib, prec):
    shapes = [(256, 512), (640, 384)]
    ts, refs = [], []
    for i, (r, c) in enumerate(shapes):
        raw, x = _normal(r, c, 1.0, "bf16", (5, i))
        ts.append(upload(raw, "bf16"))
        refs.append(orc.orthogonalize(x, 5, "gram", None, 1e-7))
    lib.dmuon_orthogonalize(ts, ts, ns_precision=prec)   # in place
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        # bf16 output rounding adds at most 2^-9 relative
        assert rel(f64(ts[i]), refs[i]) <= NS_TOL[prec] + 4e-3, shapes[i]


@pytest.mark.parametrize("prec", ["bf16", "f32"])
@pytest.mark.parametrize("coeffs", [(0.0, 1.0, 0.0), (0.0, 0.0, 1.0), (1.5, -0.5, 0.0)],
                         ids=["XXtX", "A2X", "cubic"])
def test_single_products(lib, prec, coeffs, gemm_tile):
    """One iteration with chosen coefficients isolates single products:
    (0,1,0) gives X X^T X, (0,0,1) gives (X X^T)^2 X."""
    shapes = [(256, 512), (384, 128), (1000, 1500)]
    inputs, refs = [], []
    for i, (r, c) in enumerate(shapes):
        raw, x = _normal(r, c, 1.0, "f32", (6, i))
        inputs.append(upload(raw, "f32"))
        refs.append({b: orc.orthogonalize(x, 1, b, [coeffs], 1e-7) for b in ("gram", "direct")})
    for backend in ("gram", "direct"):
        outs = [torch.empty_like(t) for t in inputs]
        lib.dmuon_orthogonalize(inputs, outs, ns_steps=1, ns_coeffs=[coeffs], ns_backend=backend,
                                ns_precision=prec)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert rel(f64(outs[i]), refs[i][backend]) <= NS_TOL[prec], (backend, shapes[i])


def test_orthogonalize_coefficient_table(lib):
    table = [(3.0, -3.2, 1.2), (2.0, -1.5, 0.5), (1.5, -0.5, 0.0)]
    raw, x = _normal(300, 900, 1.0, "f32", (7,))
    inp = upload(raw, "f32")
    for prec in ("bf16", "f32"):
        out = torch.empty_like(inp)
        lib.dmuon_orthogonalize([inp], [out], ns_steps=3, ns_coeffs=table, ns_precision=prec)
        torch.cuda.synchronize()
        ref = orc.orthogonalize(x, 3, "gram", table, 1e-7)
        assert rel(f64(out), ref) <= NS_TOL[prec]


def test_orthogonalize_degenerate(lib):
    # zero input -> zero output, no NaN
    z = torch.zeros(256, 512, device=DEV)
    out = torch.full_like(z, 7.0)
    lib.dmuon_orthogonalize([z], [out])
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    # ns_steps = 0 -> the normalised input
    raw, x = _normal(200, 300, 3.0, "f32", (8,))
    t = upload(raw, "f32")
    for prec in ("bf16", "f32"):
        o = torch.empty_like(t)
        lib.dmuon_orthogonalize([t], [o], ns_steps=0, ns_precision=prec)
        torch.cuda.synchronize()
        tol = 4e-3 if prec == "bf16" else 1e-6
        assert rel(f64(o), x / (np.linalg.norm(x) + 1e-7)) <= tol
    # rank one: the closed form is phi_5(||G||/(||G||+eps)) along the rank-one
    # direction.  Rounding the input adds noise directions with tiny singular
    # values, which the iteration is built to amplify (up to a^5 ~ 485x), so
    # the component along u v^T is checked against the closed form and the
    # rest against that amplification bound.
    u = np.random.default_rng(1).standard_normal(300)
    v = np.random.default_rng(2).standard_normal(500)
    g = np.outer(u, v).astype(np.float32)
    t = torch.from_numpy(g).to(DEV)
    uh, vh = u / np.linalg.norm(u), v / np.linalg.norm(v)
    nrm = float(np.linalg.norm(g.astype(np.float64)))
    expect = orc.orthogonalize(np.array([[nrm]]), 5, "direct", None, 1e-7)[0, 0]
    a5 = 3.4445 ** 5
    for prec, unit in (("bf16", 2.0 ** -8), ("f32", 2.0 ** -23)):
        o = torch.empty_like(t)
        lib.dmuon_orthogonalize([t], [o], ns_precision=prec)
        torch.cuda.synchronize()
        og = f64(o)
        par = float(uh @ og @ vh)
        assert abs(par - expect) <= NS_TOL[prec] * abs(expect), (prec, par, expect)
        resid = np.linalg.norm(og - par * np.outer(uh, vh))
        assert resid <= min(a5 * unit * np.sqrt(300), 1.2 * np.sqrt(299)), (prec, resid)
