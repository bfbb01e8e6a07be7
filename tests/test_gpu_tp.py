"""GPU parity of Newton-Schulz on tensor-parallel shards
(dmuon_orthogonalize_sharded) against the sharded oracle, through the C ABI.

Tolerances: the NS tolerances of the unsharded path, on every matrix (the
relative Frobenius error of its joined output): <= 2e-2 with bf16 products,
<= 1e-4 with fp32 products; with ns_steps = 0 the output is the input scaled
by the global norm, <= 1e-6 (fp32) or within one bf16 ulp.
"""
import numpy as np
import pytest
import torch

import dmuon_inputs as di
from oracle import muon as orc
from oracle import tp_gram as otp
from tests.gpu_helpers import DEV, assert_bf16_close, f64, rel, upload

pytestmark = pytest.mark.gpu

NS_TOL = {"bf16": 2e-2, "f32": 1e-4}

# (rows, cols, split, shard sizes along the split): the Gram form (D >= 2d)
# for column and row blocks, the direct form with a Gram sum per iteration
# (near-square), a Gram matrix over the longer side, a single shard, ragged
# tails of several tiles
CASES = [
    (256, 1000, 1, (300, 500, 200)),
    (1000, 256, 0, (128, 640, 232)),
    (400, 500, 1, (250, 250)),
    (600, 200, 1, (120, 80)),
    (300, 700, 1, (700,)),
    (130, 1100, 1, (1, 555, 544)),
    (1500, 520, 0, (500, 500, 500)),
]


def _inputs(cases, dtype, seed):
    mats, exact = [], []
    for i, (r, c, split, sizes) in enumerate(cases):
        raw, u = di.normal_matrix(r, c, 1.0, dtype, seed=seed, tag=(70, i))
        parts_raw = otp.split_matrix(raw, split, sizes)
        parts = otp.split_matrix(u, split, sizes)
        mats.append([upload(np.ascontiguousarray(p), dtype) for p in parts_raw])
        exact.append(parts)
    return mats, exact


def _check(got_parts, ref_parts, split, tol, what):
    got = otp.join_shards([f64(t) for t in got_parts], split)
    ref = otp.join_shards(ref_parts, split)
    err = rel(got, ref)
    assert err <= tol, (what, err)
    return err


@pytest.mark.parametrize("backend", ["gram", "direct"])
@pytest.mark.parametrize("prec", ["bf16", "f32"])
def test_sharded_parity(lib, gemm_tile, backend, prec):
    io = "f32" if prec == "f32" else "bf16"
    ins, exact = _inputs(CASES, io, seed=1)
    outs = [[torch.full_like(t, float("nan")) for t in mat] for mat in ins]
    splits = [c[2] for c in CASES]
    lib.dmuon_orthogonalize_sharded(ins, outs, splits, ns_backend=backend, ns_precision=prec)
    torch.cuda.synchronize()
    for i, (r, c, split, sizes) in enumerate(CASES):
        ref = otp.orthogonalize_sharded(exact[i], split, 5, backend)
        _check(outs[i], ref, split, NS_TOL[prec], f"{(r, c, split, sizes)} {backend} {prec}")


def test_sharded_matches_unsharded_call(lib):
    """The sharded call and dmuon_orthogonalize of the joined matrix agree
    about as closely as each agrees with the oracle."""
    cases = [(256, 1000, 1, (300, 500, 200)), (400, 500, 1, (250, 250))]
    ins, exact = _inputs(cases, "bf16", seed=2)
    outs = [[torch.empty_like(t) for t in mat] for mat in ins]
    lib.dmuon_orthogonalize_sharded(ins, outs, [c[2] for c in cases])
    joined = [torch.cat(mat, dim=1 if c[2] == 1 else 0).contiguous() for mat, c in zip(ins, cases)]
    whole = [torch.empty_like(t) for t in joined]
    lib.dmuon_orthogonalize(joined, whole)
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        a = otp.join_shards([f64(t) for t in outs[i]], c[2])
        b = f64(whole[i])
        ref = otp.join_shards(otp.orthogonalize_sharded(exact[i], c[2], 5, "gram"), c[2])
        assert rel(a, b) <= 2 * NS_TOL["bf16"], c
        assert rel(b, ref) <= NS_TOL["bf16"], c


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_sharded_no_iterations_is_global_scaling(lib, io):
    cases = [(256, 1000, 1, (300, 500, 200)), (1000, 256, 0, (128, 640, 232))]
    ins, exact = _inputs(cases, io, seed=3)
    outs = [[torch.empty_like(t) for t in mat] for mat in ins]
    lib.dmuon_orthogonalize_sharded(ins, outs, [c[2] for c in cases], ns_steps=0, ns_precision="f32")
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        ref = otp.orthogonalize_sharded(exact[i], c[2], 0, "gram")
        for g, r in zip(outs[i], ref):
            if io == "f32":
                assert rel(f64(g), r) <= 1e-6, c
            else:
                assert_bf16_close(f64(g), orc.round_to_bf16(r), what=str(c))


def test_sharded_in_place_and_repeatable(lib):
    cases = [(256, 1000, 1, (300, 500, 200)), (400, 500, 1, (250, 250)), (600, 200, 1, (120, 80))]
    ins, _ = _inputs(cases, "bf16", seed=4)
    a = [[t.clone() for t in mat] for mat in ins]
    b = [[torch.empty_like(t) for t in mat] for mat in ins]
    lib.dmuon_orthogonalize_sharded(ins, b, [c[2] for c in cases])
    lib.dmuon_orthogonalize_sharded(a, a, [c[2] for c in cases])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        for p, q in zip(x, y):
            assert torch.equal(p, q)


def test_sharded_3b_layer_tp8(lib):
    """One 3B decoder layer with every matrix in 8 tensor-parallel shards, as
    the usual layout splits them: q, k, v, gate, up by output rows (row
    blocks), o and down by input columns (column blocks).  k and v
    (1024 x 3072 in rows of 128) form their Gram matrices over the longer
    side.  One call; one matrix of each kind against the oracle."""
    w = di.workload(1)
    split_of = {"q": 0, "k": 0, "v": 0, "gate": 0, "up": 0, "o": 1, "down": 1}
    ins, exact, splits, names = [], [], [], []
    for i, m in enumerate(w.matrices):
        kind = m.name.split(".")[-1].replace("_proj", "")
        split = split_of[kind]
        raw, u = di.normal_matrix(m.rows, m.cols, 1e-3, "bf16", seed=5, tag=(71, i))
        along = m.rows if split == 0 else m.cols
        sizes = [along // 8] * 8
        ins.append([upload(np.ascontiguousarray(p), "bf16") for p in otp.split_matrix(raw, split, sizes)])
        exact.append(otp.split_matrix(u, split, sizes))
        splits.append(split)
        names.append(kind)
    outs = [[torch.empty_like(t) for t in mat] for mat in ins]
    lib.dmuon_orthogonalize_sharded(ins, outs, splits)
    torch.cuda.synchronize()
    for kind in ("q", "k", "gate", "down"):
        i = names.index(kind)
        ref = otp.orthogonalize_sharded(exact[i], splits[i], 5, "gram")
        _check(outs[i], ref, splits[i], NS_TOL["bf16"], kind)
    for i in range(len(outs)):
        o = otp.join_shards([f64(t) for t in outs[i]], splits[i])
        assert np.isfinite(o).all(), names[i]
