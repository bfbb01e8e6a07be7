"""The seeded synthetic workloads: shapes, counts, determinism, rounding."""
import numpy as np

import dmuon_inputs as di


def test_workload_shapes():
    w1 = di.workload(1)
    assert [(m.rows, m.cols) for m in w1.matrices] == [
        (3072, 3072), (1024, 3072), (1024, 3072), (3072, 3072),
        (8192, 3072), (8192, 3072), (3072, 8192)]
    assert w1.numel == 100_663_296 and w1.steps == 10
    w2 = di.workload(2)
    assert len(w2.matrices) == 196 and w2.numel == 28 * w1.numel == 2_818_572_288
    w3 = di.workload(3)
    assert len(w3.matrices) == 28 and w3.numel == 872_415_232 and w3.weight_decay == 0.1
    w4 = di.workload(4)
    counts = np.bincount(di.ragged_shape_draw(0), minlength=7)
    assert counts.tolist() == [14, 8, 16, 13, 18, 15, 12]
    assert len(w4.matrices) == 96 and all(m.rows * m.cols > 100_000 for m in w4.matrices)
    w0 = di.workload(0)
    assert (w0.matrices[0].rows, w0.matrices[0].cols) == (256, 512) and w0.param_dtype == "f32"


def test_streams_deterministic_and_distinct():
    w = di.workload(0)
    a, ea = di.grad_at(w, 0, 0)
    b, eb = di.grad_at(w, 0, 0)
    c, _ = di.grad_at(w, 0, 1)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert abs(ea.std() - 1e-2) < 1e-3


def test_bf16_storage_rounding():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-40, np.nan])
    raw, exact = di.to_storage(x, "bf16")
    assert raw.dtype == np.uint16
    assert exact[0] == 1.0 and exact[1] == 1.0          # tie to even
    assert exact[2] == 1.0 + 4 * 2 ** -8                # tie to even (up)
    assert exact[3] == -2.5 and np.isnan(exact[5])


def test_lognormal_grad_scales():
    w = di.workload(4)
    s = np.array([di.grad_scale(w, i) for i in range(len(w.matrices))])
    assert np.all(s > 0) and 0.3 < np.std(np.log(s / 1e-3)) < 2.0
