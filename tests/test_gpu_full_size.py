"""GPU parity at the full sizes of the benchmark workloads, over each
workload's whole step count, in the launch configuration the benchmark
times: every matrix of a workload in one dmuon_step call per step with the
default tile choice, inputs generated on the device from seeded generators.

Checked, relative Frobenius error unless stated:
  * every step, every matrix: the momentum buffer against an fp64
    recomputation of the recurrence M <- mu*M + G from the exact gradient
    bytes (<= 1e-6); the sampled matrices (one of every distinct shape, both
    orientations where the workload holds both) also against the oracle's
    own recurrence on the host;
  * at the first and the last step:
      - the step's NS input U (the momentum stage run on copies of the
        buffers, in fp32) against the oracle's U (<= 1e-6),
      - the NS output O of that U, computed by dmuon_orthogonalize over the
        whole batch (the same plan, hence the same launches and tiles as
        the step), against the oracle's NS of the oracle's own U, directly:
        <= 2e-2 with bf16 products, <= 1e-4 with fp32 products, no rounding
        allowance,
      - the parameter after the step (bf16, written by the fused update of
        the last product) against the oracle's update applied to the
        parameter before the step: the NS tolerance plus the norm of half a
        bf16 ulp of the result (the one rounding the step makes),
      - every matrix: O finite, spectral norm at most
        max_[0,1] phi_5 = 1.2024 (plus 5 %), mean squared singular value
        ||O||_F^2 / m in [0.45, 1.45] (Gaussian inputs give 0.73-0.89).
Measured errors go to the file named by DMUON_PARITY_LOG (JSON lines), if set.
"""
import json
import os
import time

import numpy as np
import pytest
import torch

import dmuon_inputs as di
from oracle import muon as orc
from tests.gpu_helpers import DEV, check_param_step, f64, rel

pytestmark = pytest.mark.gpu

NS_TOL = {"bf16": 2e-2, "f32": 1e-4}
PHI5_MAX = 1.2024     # max of the five-fold default quintic on [0, 1]


def _log(rec: dict) -> None:
    path = os.environ.get("DMUON_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def _spectral_norm(o: torch.Tensor, iters: int = 30) -> float:
    v = torch.ones(o.shape[1], dtype=torch.float32, device=o.device)
    v /= v.norm()
    s = 0.0
    for _ in range(iters):
        u = o @ v
        v = o.t() @ u
        s = float(v.norm().sqrt())
        v /= v.norm()
    return s


def _distinct_shapes(w: di.Workload):
    seen, idx = set(), []
    for i, m in enumerate(w.matrices):
        if (m.rows, m.cols) not in seen:
            seen.add((m.rows, m.cols))
            idx.append(i)
    return idx


def _grads(w: di.Workload, step: int, seed_base: int):
    out = []
    for i, m in enumerate(w.matrices):
        g = torch.empty(m.rows, m.cols, dtype=torch.bfloat16, device=DEV)
        di.torch_normal_(g, di.grad_scale(w, i), seed=seed_base + 100000 * (step + 1) + i)
        out.append(g)
    return out


def _run_workload(w: di.Workload, hp: dict, seed_base: int, lib, sampled=None):
    prec = hp["ns_precision"]
    tol = NS_TOL[prec]
    sampled = _distinct_shapes(w) if sampled is None else sampled
    params, moms = [], []
    for i, m in enumerate(w.matrices):
        p = torch.empty(m.rows, m.cols, dtype=torch.bfloat16, device=DEV)
        di.torch_normal_(p, w.param_std, seed=seed_base + i)
        params.append(p)
        moms.append(torch.zeros(m.rows, m.cols, dtype=torch.float32, device=DEV))
    shapes = [(m.rows, m.cols) for m in w.matrices]
    ws = torch.empty(lib.dmuon_step_workspace_size(params, params, moms, **hp), dtype=torch.uint8, device=DEV)
    assert ws.numel() == lib.dmuon_orthogonalize_workspace_size(shapes, **hp)
    m_dev64 = [torch.zeros(r, c, dtype=torch.float64, device=DEV) for r, c in shapes]   # recurrence, all
    m_host = {i: np.zeros(shapes[i]) for i in sampled}                                   # oracle, sampled
    checked = {0, w.steps - 1}
    tag = f"{w.name} {hp['ns_backend']}/{prec}"
    for step in range(w.steps):
        grads = _grads(w, step, seed_base)
        g_host = {i: f64(grads[i]) for i in sampled}
        u_ref = {}
        for i in sampled:
            m_host[i], u_ref[i] = orc.momentum_update(m_host[i], g_host[i], hp["momentum"], hp["nesterov"])
        o_gpu = u_gpu = w_before = None
        if step in checked:
            # the step's own NS input, then its NS output through the same plan
            mom_copy = [m.clone() for m in moms]
            u_gpu = [torch.empty(min(r, c), max(r, c), dtype=torch.float32, device=DEV) for r, c in shapes]
            sumsq = torch.empty(len(shapes), dtype=torch.float64, device=DEV)
            lib.dmuon_momentum(grads, mom_copy, u_gpu, sumsq, momentum=hp["momentum"], nesterov=hp["nesterov"],
                               workspace=ws)
            del mom_copy
            o_gpu = [torch.empty_like(u) for u in u_gpu]
            lib.dmuon_orthogonalize(u_gpu, o_gpu, workspace=ws, **hp)
            w_before = {i: f64(params[i]) for i in sampled}
        t0 = time.time()
        lib.dmuon_step(params, grads, moms, workspace=ws, **hp)
        torch.cuda.synchronize()
        t_gpu = time.time() - t0

        # momentum of every matrix: fp64 recurrence from the exact gradient bytes
        worst_m = 0.0
        for i in range(len(shapes)):
            m_dev64[i].mul_(hp["momentum"]).add_(grads[i].double())
            e = float((moms[i].double() - m_dev64[i]).norm() / m_dev64[i].norm())
            worst_m = max(worst_m, e)
            assert e <= 1e-6, (tag, step, i, e)
        for i in sampled:
            assert rel(f64(moms[i]), m_host[i]) <= 1e-6, (tag, step, i)
        print(f"{tag} step {step}: GPU {t_gpu:.2f}s, momentum worst rel err {worst_m:.2e}", flush=True)
        _log({"workload": w.index, "backend": hp["ns_backend"], "precision": prec, "step": step,
              "check": "momentum_all", "max_rel_err": worst_m})
        if step not in checked:
            del grads
            continue

        # properties of every matrix's NS output
        for i, (r, c) in enumerate(shapes):
            o = o_gpu[i]
            assert torch.isfinite(o).all(), (tag, step, i)
            msq = float((o * o).sum()) / min(r, c)
            sn = _spectral_norm(o)
            assert 0.45 <= msq <= 1.45, (tag, step, i, msq)
            assert sn <= PHI5_MAX * 1.05, (tag, step, i, sn)
        # the sampled matrices against the oracle
        for i in sampled:
            m = w.matrices[i]
            tall = m.rows > m.cols
            uw_ref = u_ref[i].T if tall else u_ref[i]
            e_u = rel(f64(u_gpu[i]), uw_ref)
            assert e_u <= 1e-6, (tag, step, m.name, e_u)
            t1 = time.time()
            o_ref_w = orc.orthogonalize(uw_ref, hp["ns_steps"], hp["ns_backend"], None, hp["eps"])
            e_o = rel(f64(o_gpu[i]), o_ref_w)
            o_ref = o_ref_w.T if tall else o_ref_w
            w_ref = orc.apply_update(w_before[i], o_ref, hp["lr"], hp["weight_decay"])
            e_w = check_param_step(f64(params[i]), w_before[i], w_ref, "bf16", tol, prec,
                                   what=f"{tag} {m.name}", elementwise=False)
            print(f"{tag} step {step} {m.name} {m.rows}x{m.cols}: U {e_u:.1e}, O {e_o:.3e}, "
                  f"update {e_w:.3e} (oracle {time.time() - t1:.1f}s)", flush=True)
            _log({"workload": w.index, "backend": hp["ns_backend"], "precision": prec, "step": step,
                  "matrix": m.name, "shape": [m.rows, m.cols], "u_rel_err": e_u, "o_rel_err": e_o,
                  "update_rel_err": e_w})
            assert e_o <= tol, (tag, step, m.name, e_o)
        del grads, u_gpu, o_gpu
    del params, moms, m_dev64, ws
    torch.cuda.empty_cache()


def test_full_decoder_layer_ten_steps(lib):
    """One 3B decoder layer, ten steps; every one of its seven matrices is
    checked against the oracle at the first and the last step."""
    w = di.workload(1)
    _run_workload(w, w.hparams(), 6000, lib, sampled=list(range(len(w.matrices))))


def test_full_3b_stack_gram(lib):
    """28-layer 3B stack, 196 matrices, Gram backend, five steps."""
    w = di.workload(2)
    _run_workload(w, w.hparams(ns_backend="gram"), 7000, lib)


def test_full_3b_stack_direct(lib):
    """28-layer 3B stack, standard-form backend, five steps."""
    w = di.workload(2)
    _run_workload(w, w.hparams(ns_backend="direct"), 8000, lib)


def test_full_8b_layers_weight_decay(lib):
    """8B layers 0-3 (28 matrices, up to 14336 x 4096) with weight decay 0.1, five steps."""
    w = di.workload(3)
    _run_workload(w, w.hparams(), 9000, lib)


@pytest.mark.parametrize("prec", ["bf16", "f32"])
def test_full_ragged_lognormal(lib, prec):
    """96 ragged matrices, log-normal gradient scales, both NS precisions, three steps."""
    w = di.workload(4)
    _run_workload(w, w.hparams(ns_precision=prec), 10000, lib)
