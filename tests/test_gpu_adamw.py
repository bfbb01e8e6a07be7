"""GPU parity of the fused AdamW step (dmuon_adamw_step) against the oracle.

Tolerances, derived from the fp32 evaluation (each of m, v and the parameter
is a short chain of fp32 products, one fused multiply-add, a square root and
a division, each rounded once):
  * first step (identical inputs on both sides): every element of m within
    4 ulp-units of 2^-24 (|beta1 m| + |(1-beta1) g|), of v within 6 units of
    2^-24 (|beta2 v| + |(1-beta2) g^2|); an fp32 parameter within
    4 * 2^-24 (|p| + 8 |update|);
  * later steps (each side carries its own state): the relative Frobenius
    error of m, v and of the fp32 parameter's change <= 1e-6;
  * bf16 parameters: every element within one bf16 ulp of the oracle's
    rounded value (plus the fp32 evaluation slack above), >= 99.9 % equal.
"""
import numpy as np
import pytest
import torch

import dmuon_inputs as di
from oracle import adamw as oad
from tests.gpu_helpers import DEV, assert_bf16_close, f64, rel, upload

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
# sizes below, at and past the 8192-element chunk, 2-D, one element
SIZES = [(1000,), (8192,), (8193,), (33, 7), (70001,), (1,), (3, 16384), (5,)]
GROUPS = [dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01),
          dict(lr=3e-3, betas=(0.8, 0.95), eps=1e-6, weight_decay=0.1)]


def _ref_hp(g):
    return dict(lr=g["lr"], beta1=g["betas"][0], beta2=g["betas"][1], eps=g["eps"], weight_decay=g["weight_decay"])


def _draw(shape, std, dtype, tag):
    raw, ex = di.normal_matrix(int(np.prod(shape)), 1, std, dtype, seed=0, tag=tag)
    return upload(raw.reshape(shape), dtype), ex.reshape(shape)


def _check_first_step(p_got, m_got, v_got, p_in, g, hp, pdt, what):
    p_ref, m_ref, v_ref = oad.adamw_step(p_in, g, 0 * g, 0 * g, 1, **hp)
    b1, b2 = hp["beta1"], hp["beta2"]
    assert np.all(np.abs(m_got - m_ref) <= 4 * U * ((1 - b1) * np.abs(g)) + 1e-45), what
    assert np.all(np.abs(v_got - v_ref) <= 6 * U * ((1 - b2) * g * g) + 1e-45), what
    upd = np.abs(p_in * (1 - hp["lr"] * hp["weight_decay"]) - p_ref)
    slack = 4 * U * (np.abs(p_in) + 8 * upd)
    if pdt == "f32":
        assert np.all(np.abs(p_got - p_ref) <= slack + np.spacing(np.abs(p_ref).astype(np.float32))), what
    else:
        assert_bf16_close(p_got, oad.store(p_ref, "bf16"), slack=slack, what=what)


@pytest.mark.parametrize("pdt,gdt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16")])
def test_adamw_parity_three_steps(lib, pdt, gdt):
    n = len(SIZES)
    gidx = [i % 2 for i in range(n)]
    params, p_ref = [], []
    for i, s in enumerate(SIZES):
        t, ex = _draw(s, 0.02, pdt, (80, i))
        params.append(t)
        p_ref.append(ex)
    p0 = [x.copy() for x in p_ref]
    ms = [torch.zeros(s, dtype=torch.float32, device=DEV) for s in SIZES]
    vs = [torch.zeros(s, dtype=torch.float32, device=DEV) for s in SIZES]
    m_ref = [np.zeros(s) for s in SIZES]
    v_ref = [np.zeros(s) for s in SIZES]
    for step in range(1, 4):
        grads, g_ex = [], []
        for i, s in enumerate(SIZES):
            t, ex = _draw(s, 1e-3 * (i + 1), gdt, (81, i, step))
            grads.append(t)
            g_ex.append(ex)
        groups = [dict(g, step=step) for g in GROUPS]
        lib.dmuon_adamw_step(params, grads, ms, vs, step=step, groups=groups, group_index=gidx)
        torch.cuda.synchronize()
        for i in range(n):
            hp = _ref_hp(GROUPS[gidx[i]])
            what = f"step {step} tensor {i} {SIZES[i]} {pdt}/{gdt}"
            if step == 1:
                _check_first_step(f64(params[i]), f64(ms[i]), f64(vs[i]), p_ref[i], g_ex[i], hp, pdt, what)
            p_new, m_ref[i], v_ref[i] = oad.adamw_step(p_ref[i], g_ex[i], m_ref[i], v_ref[i], step, **hp)
            p_ref[i] = oad.store(p_new, pdt)
            if step > 1:
                assert rel(f64(ms[i]), m_ref[i]) <= 1e-6, what
                assert rel(f64(vs[i]), v_ref[i]) <= 1e-6, what
                if pdt == "f32":
                    assert rel(f64(params[i]) - p0[i], p_ref[i] - p0[i]) <= 1e-6, what
                else:
                    upd = np.abs(p_new - p_ref[i]) + hp["lr"]
                    assert_bf16_close(f64(params[i]), p_ref[i], min_exact=0.99,
                                      slack=4 * U * (np.abs(p_ref[i]) + 8 * upd), what=what)


def test_adamw_unaligned_skip_and_neighbours(lib):
    """Tensors at odd element offsets take the scalar path; the elements
    around them and a tensor with no gradient stay untouched."""
    store = torch.zeros(3 * 9000 + 5, dtype=torch.bfloat16, device=DEV)
    views = [store[1:9001], store[9002:18002], store[18003:27003]]
    vals = []
    rng = np.random.default_rng(4)
    for v in views:
        raw, ex = di.to_storage(rng.standard_normal(v.numel()) * 0.02, "bf16")
        v.copy_(upload(raw, "bf16"))
        vals.append(ex)
    gstore = torch.zeros(3 * 9000 + 3, dtype=torch.float32, device=DEV)
    gviews = [gstore[1:9001], gstore[9001:18001], gstore[18002:27002]]
    gvals = []
    for gv in gviews:
        raw, ex = di.to_storage(rng.standard_normal(gv.numel()) * 1e-3, "f32")
        gv.copy_(upload(raw, "f32"))
        gvals.append(ex)
    ms = [torch.zeros(9000, dtype=torch.float32, device=DEV) for _ in views]
    vs = [torch.zeros(9000, dtype=torch.float32, device=DEV) for _ in views]
    skipped = torch.full((100,), 0.5, dtype=torch.float32, device=DEV)
    sm, sv = torch.zeros_like(skipped), torch.zeros_like(skipped)
    lib.dmuon_adamw_step(views + [skipped], gviews + [None], ms + [sm], vs + [sv], step=1)
    torch.cuda.synchronize()
    hp = oad.DEFAULTS
    for i in range(3):
        _check_first_step(f64(views[i]), f64(ms[i]), f64(vs[i]), vals[i], gvals[i], hp, "bf16", f"view {i}")
    assert store[0].item() == 0.0 and store[9001].item() == 0.0 and store[-1].item() == 0.0
    assert torch.all(skipped == 0.5) and torch.all(sm == 0) and torch.all(sv == 0)


def test_adamw_deterministic(lib):
    a = [_draw(s, 0.02, "bf16", (82, i))[0] for i, s in enumerate(SIZES)]
    b = [t.clone() for t in a]
    g = [_draw(s, 1e-3, "bf16", (83, i))[0] for i, s in enumerate(SIZES)]
    st = [[torch.zeros(s, dtype=torch.float32, device=DEV) for s in SIZES] for _ in range(4)]
    lib.dmuon_adamw_step(a, g, st[0], st[1], step=1)
    lib.dmuon_adamw_step(b, g, st[2], st[3], step=1)
    torch.cuda.synchronize()
    for x, y in zip(a + st[0] + st[1], b + st[2] + st[3]):
        assert torch.equal(x, y)


def test_adamw_3b_symmetric_group(lib):
    """The AdamW group of a 3B-shaped model: the 128256 x 3072 embedding and
    57 RMSNorm weights of 3072, bf16 parameters and gradients, two steps in
    one call each; 2^20 sampled elements of the embedding and every norm
    against the oracle's own trajectory."""
    shapes = [(128256, 3072)] + [(3072,)] * 57
    params, grads, ms, vs = [], [], [], []
    for i, s in enumerate(shapes):
        p = torch.empty(s, dtype=torch.bfloat16, device=DEV)
        di.torch_normal_(p, 0.02, seed=40000 + i)
        params.append(p)
        ms.append(torch.zeros(s, dtype=torch.float32, device=DEV))
        vs.append(torch.zeros(s, dtype=torch.float32, device=DEV))
    rng = np.random.default_rng(6)
    idx = np.unique(rng.integers(0, shapes[0][0] * shapes[0][1], size=1 << 20))
    flat0 = params[0].view(-1)
    p_ref = [f64(flat0[torch.from_numpy(idx).to(DEV)])] + [f64(p) for p in params[1:]]
    m_ref = [np.zeros_like(x) for x in p_ref]
    v_ref = [np.zeros_like(x) for x in p_ref]
    hp = oad.DEFAULTS
    for step in (1, 2):
        grads = []
        for i, s in enumerate(shapes):
            g = torch.empty(s, dtype=torch.bfloat16, device=DEV)
            di.torch_normal_(g, 1e-3, seed=50000 + 100 * step + i)
            grads.append(g)
        g_s = [f64(grads[0].view(-1)[torch.from_numpy(idx).to(DEV)])] + [f64(g) for g in grads[1:]]
        lib.dmuon_adamw_step(params, grads, ms, vs, step=step)
        torch.cuda.synchronize()
        got = [f64(params[0].view(-1)[torch.from_numpy(idx).to(DEV)])] + [f64(p) for p in params[1:]]
        got_m = [f64(ms[0].view(-1)[torch.from_numpy(idx).to(DEV)])] + [f64(m) for m in ms[1:]]
        for i in range(len(shapes)):
            p_new, m_ref[i], v_ref[i] = oad.adamw_step(p_ref[i], g_s[i], m_ref[i], v_ref[i], step, **hp)
            p_ref[i] = oad.store(p_new, "bf16")
            upd = np.abs(p_new - p_ref[i]) + hp["lr"]
            assert_bf16_close(got[i], p_ref[i], min_exact=0.99, slack=4 * U * (np.abs(p_ref[i]) + 8 * upd),
                              what=f"step {step} tensor {i}")
            assert rel(got_m[i], m_ref[i]) <= 1e-6, (step, i)
