"""GPU parity of the whole step (dmuon_step) against the oracle, plus the
properties the step must keep: matrix independence, skipped matrices,
determinism and bit-identical resume.

Parity measures (relative Frobenius error):
  momentum buffer after every step        <= 1e-6
  parameter change W_new - W_old          <= 2e-2 (bf16 NS) / 1e-4 (fp32 NS)
"""
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
    """A batch of differently shaped matrices over three steps.  Checked
    after every step: the momentum against the oracle's own recurrence
    (relative error <= 1e-6), and each parameter against the oracle's update
    of the GPU's own parameter before the step with the oracle's NS output
    of the oracle's own NS input: fp32 parameters to the NS tolerance, bf16
    parameters to the NS tolerance plus half a bf16 ulp of the result (the
    one rounding of the step), and with fp32 products every element within
    one bf16 ulp of the oracle's rounded value (99 % equal)."""
    specs = RAGGED_SPECS[batch]
    rng = np.random.default_rng(11)
    params, moms, m_ref = [], [], []
    for i, (r, c, dt) in enumerate(specs):
        raw, _ = di.normal_matrix(r, c, 0.02, dt, seed=0, tag=(20, i))
        params.append(upload(raw, dt))
        moms.append(torch.zeros(r, c, dtype=torch.float32, device=DEV))
        m_ref.append(np.zeros((r, c)))
    hp = dict(lr=0.02, momentum=0.95, nesterov=True, ns_steps=5, weight_decay=0.1,
              ns_backend="gram", ns_precision=prec)
    for step in range(3):
        gs = [di.normal_matrix(r, c, 1e-3 * float(np.exp(rng.standard_normal())), dt, seed=0,
                               tag=(21, i, step)) for i, (r, c, dt) in enumerate(specs)]
        grads = [upload(raw, dt) for (raw, _), (_, _, dt) in zip(gs, specs)]
        w_old = [f64(p) for p in params]
        lib.dmuon_step(params, grads, moms, **hp)
        torch.cuda.synchronize()
        for i, (r, c, dt) in enumerate(specs):
            w_ref, m_ref[i], _, _ = orc.muon_step(w_old[i], gs[i][1], m_ref[i], ns_backend="gram",
                                                  weight_decay=0.1, param_dtype="f32")
            assert rel(f64(moms[i]), m_ref[i]) <= 1e-6, (step, i)
            got = f64(params[i])
            assert np.isfinite(got).all()
            err = check_param_step(got, w_old[i], w_ref, dt, NS_TOL[prec], prec,
                                   what=f"step {step} {r}x{c} {dt}")
            print(f"step {step} {r}x{c} {dt} ns={prec} tile={gemm_tile}: update rel err {err:.3e}")


def test_step_on_side_stream(lib):
    """A step on a stream other than the current one, with the workspace
    allocated by the binding, while the current stream allocates and writes
    memory before anything waits for the step: the result is bit-identical
    to the same step on the current stream."""
    shapes = [(2048, 8192), (8192, 2048), (3072, 3072), (1024, 4096)]
    def init():
        ps = [upload(di.normal_matrix(r, c, 0.02, "bf16", 0, (50, i))[0], "bf16") for i, (r, c) in enumerate(shapes)]
        ms = [torch.zeros(r, c, dtype=torch.float32, device=DEV) for r, c in shapes]
        return ps, ms
    grads = [upload(di.normal_matrix(r, c, 1e-3, "bf16", 0, (51, i))[0], "bf16") for i, (r, c) in enumerate(shapes)]
    pa, ma = init()
    lib.dmuon_step(pa, grads, ma)
    torch.cuda.synchronize()
    nbytes = lib.dmuon_step_workspace_size(pa, grads, ma)
    pb, mb = init()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    lib.dmuon_step(pb, grads, mb, stream=side)       # workspace allocated by the binding
    junk = [torch.full((nbytes // 4 + 4096,), 7, dtype=torch.uint8, device=DEV) for _ in range(4)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    for i in range(len(shapes)):
        assert torch.equal(pa[i], pb[i]) and torch.equal(ma[i], mb[i]), i


def test_queued_split_steps_do_not_block_host(lib):
    """Many steps of a batch that runs as two stream groups, enqueued without
    a synchronisation: the host must not wait on the GPU while enqueueing
    (it once did, about 2.5 ms per step, behind the launch-table copies), and
    the result is bit-identical to the same steps synchronised one by one."""
    import time
    shapes = [(3072, 3072)] * 4
    assert len(lib.dmuon_plan_describe(shapes)["stream_groups"]) == 2
    grads = [upload(di.normal_matrix(r, c, 1e-3, "bf16", 0, (60, i))[0], "bf16") for i, (r, c) in enumerate(shapes)]
    def init():
        ps = [upload(di.normal_matrix(r, c, 0.02, "bf16", 0, (61, i))[0], "bf16") for i, (r, c) in enumerate(shapes)]
        return ps, [torch.zeros(r, c, dtype=torch.float32, device=DEV) for r, c in shapes]
    ws = torch.empty(lib.dmuon_step_workspace_size(*init()[:1], grads, init()[1]), dtype=torch.uint8, device=DEV)
    pa, ma = init()
    for _ in range(3):                                # warm-up: plans, images, streams
        lib.dmuon_step(pa, grads, ma, workspace=ws)
    torch.cuda.synchronize()
    pa, ma = init()
    pb, mb = [p.clone() for p in pa], [m.clone() for m in ma]
    steps = 30
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    t0 = time.perf_counter()
    for _ in range(steps):
        lib.dmuon_step(pa, grads, ma, workspace=ws)
    host_ms = (time.perf_counter() - t0) * 1e3
    end.record()
    torch.cuda.synchronize()
    gpu_ms = start.elapsed_time(end)
    print(f"{steps} queued steps: host {host_ms:.2f} ms, GPU {gpu_ms:.2f} ms")
    assert host_ms < 0.5 * gpu_ms, (host_ms, gpu_ms)
    for _ in range(steps):
        lib.dmuon_step(pb, grads, mb, workspace=ws)
        torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(pa[i], pb[i]) and torch.equal(ma[i], mb[i]), i


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
