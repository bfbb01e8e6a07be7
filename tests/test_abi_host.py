"""Host-side checks of the C-ABI library: it loads, exports every symbol the
header declares, and its host-only logic (argument checks, workspace sizing,
the launch planner) behaves.  No kernel is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dmuon.h")


@pytest.fixture(scope="module")
def dm():
    import matrix_optimizer_step_owned_amd as dm
    return dm


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dmuon_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(dm):
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(dm._lib, n), n
        assert n in dm.EXPORTS, f"binding does not wrap {n}"
    assert set(dm.EXPORTS) == set(names)


def test_struct_layout_matches_header(dm):
    assert ctypes.sizeof(dm.dmuon_matrix_t) == 48
    assert ctypes.sizeof(dm.dmuon_hparams_t) == 64
    assert dm.dmuon_hparams_t.eps.offset == 56


def test_defaults_match_pages(dm):
    import json
    pages = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_hyperparameters.json")))
    d = dm.dmuon_hparams_default()
    for k in ("lr", "momentum", "nesterov", "ns_steps", "weight_decay", "ns_backend"):
        assert d[k] == pages[k], k
    assert d["eps"] == 1e-7


def test_status_strings(dm):
    for code in (0, -1, -2, -3, -4, -5):
        assert dm.dmuon_status_string(code)
    assert dm.dmuon_status_string(-99) == "unknown status"
    info = dm.dmuon_backend_info()
    assert info["arch"] == "gfx950" and "gram_rule" in info


def _mats(dm, shapes, dtype=1, grad=True):
    arr = (dm.dmuon_matrix_t * len(shapes))()
    addr = 1 << 20
    for i, (r, c) in enumerate(shapes):
        m = arr[i]
        m.rows, m.cols = r, c
        es = 4 if dtype == 0 else 2
        m.param = addr; addr += r * c * es + 4096
        m.grad = addr if grad else None; addr += r * c * es + 4096
        m.momentum = addr; addr += r * c * 4 + 4096
        m.param_dtype = m.grad_dtype = dtype
    return arr


def _hp(dm, **kw):
    h, keep = dm._hparams(**kw)
    return h, keep


def test_argument_errors_before_launch(dm):
    """Invalid arguments return a status before any device work (these calls
    would fault if they reached a kernel: the pointers are fake)."""
    lib = dm._lib
    h, _ = _hp(dm)
    mats = _mats(dm, [(256, 512)])
    ws = 1 << 40
    def call(mats=mats, n=1, hp=h, ws=ws, wsb=1 << 40):
        return lib.dmuon_step(mats, n, ctypes.byref(hp), ws, wsb, None)
    assert call(n=-1) == dm.DMUON_ERR_INVALID_ARG
    bad = _mats(dm, [(0, 512)])
    assert call(mats=bad) == dm.DMUON_ERR_INVALID_ARG
    bad = _mats(dm, [(256, 512)])
    bad[0].param_dtype = 7
    assert call(mats=bad) == dm.DMUON_ERR_UNSUPPORTED
    bad = _mats(dm, [(256, 512)])
    bad[0].momentum = None
    assert call(mats=bad) == dm.DMUON_ERR_INVALID_ARG
    for kw in (dict(ns_steps=17), dict(ns_steps=-1), dict(lr=float("nan")), dict(eps=-1.0),
               dict(ns_backend=5), dict(ns_precision=3), dict(momentum=float("inf")),
               dict(ns_coeffs=[1.0, 2.0]), dict(ns_coeffs=[1.0, 2.0, float("nan")])):
        hh, _k = _hp(dm, **kw)
        assert call(hp=hh) == dm.DMUON_ERR_INVALID_ARG, kw
    need = lib.dmuon_step_workspace_size(mats, 1, ctypes.byref(h))
    assert need > 0
    assert call(ws=None) == dm.DMUON_ERR_WORKSPACE
    assert call(wsb=need - 1) == dm.DMUON_ERR_WORKSPACE
    assert call(ws=ws + 8, wsb=need) == dm.DMUON_ERR_INVALID_ARG   # misaligned
    # aliasing: two matrices share a param; workspace overlapping a grad
    two = _mats(dm, [(256, 512), (256, 512)])
    two[1].param = two[0].param
    assert lib.dmuon_step(two, 2, ctypes.byref(h), ws, 1 << 40, None) == dm.DMUON_ERR_ALIASING
    assert "overlaps" in dm.dmuon_last_error()
    assert call(ws=mats[0].grad - (mats[0].grad % 256), wsb=need + 8192) == dm.DMUON_ERR_ALIASING
    # all gradients NULL: nothing to do, no device touched
    nog = _mats(dm, [(256, 512)], grad=False)
    assert call(mats=nog, ws=None, wsb=0) == dm.DMUON_OK
    assert call(n=0, ws=None, wsb=0) == dm.DMUON_OK


def test_workspace_sizes(dm):
    lib = dm._lib
    h, _ = _hp(dm)
    # direct: 2 m x n + 2 m x m bf16; gram (n >= 2m): 2 m x n + 5 m x m
    sq = dm.dmuon_orthogonalize_workspace_size([(1024, 1024)])
    wide = dm.dmuon_orthogonalize_workspace_size([(1024, 3072)])
    assert sq >= 2 * 1024 * 1024 * 2 * 2
    # Gram form: X0, X0^T and O (m x n), A, P, T, Q0, Q1 (m x m); every
    # buffer row carries one extra 128-byte line (64 bf16 values)
    pad = 64
    gram = (2 * 1024 * (3072 + pad) + 3072 * (1024 + pad) + 5 * 1024 * (1024 + pad)) * 2
    assert gram <= wide < gram + (1 << 20)
    # direct form: X0, X0^T, X1, X1^T (m x n), A, B (m x m)
    assert sq >= (4 * 1024 * 1024 + 2 * 1024 * 1024) * 2
    f32 = dm.dmuon_orthogonalize_workspace_size([(1024, 1024)], ns_precision="f32")
    assert f32 >= 2 * sq - (1 << 20)
    assert lib.dmuon_apply_update_workspace_size(3) >= 3 * 128


def test_plan_forms_and_grouping(dm):
    import dmuon_inputs as di
    w = di.workload(1)
    shapes = [(m.rows, m.cols) for m in w.matrices]
    plan = dm.dmuon_plan_describe(shapes)
    forms = [m["form"] for m in plan["matrices"]]
    # q, o square -> direct; k, v (1024 x 3072), gate/up (tall), down -> gram
    assert forms == ["direct", "gram", "gram", "direct", "gram", "gram", "gram"]
    assert [m["tall"] for m in plan["matrices"]] == [False, False, False, False, True, True, False]
    # one launch per stage, each covering every matrix at that stage: 16 Gram
    # stages; the direct form's 15 fit inside them
    assert len(plan["launches"]) == 16
    left = [l["left_tasks"] for l in plan["launches"]]
    assert sum(1 for v in left if v) == 5 + 1   # five direct X-updates, one final Gram Q X0
    first = plan["launches"][0]
    assert first["tasks"] == 7 and first["sym_tasks"] == 7
    # tasks are ordered longest-K first inside a launch
    assert first["k_max"] == 8192 and first["k_min"] == 3072
    # executed flops: symmetric products run t(t+1)/2 of the t x t tiles
    T = plan["tile"]
    def sym(m, k): t = m // T; return 2 * (t * (t + 1) // 2) * T * T * k
    def gen(m, n, k): return 2 * m * n * k
    def direct(m, n): return 5 * (sym(m, n) + sym(m, m) + gen(m, n, m))
    def gram(m, n): return sym(m, n) + (5 + 4 + 8) * sym(m, m) + gen(m, n, m)
    expect = 2 * direct(3072, 3072) + 2 * gram(1024, 3072) + 3 * gram(3072, 8192)
    assert sum(l["flops"] for l in plan["launches"]) == expect


def test_plan_all_direct_and_small(dm):
    plan = dm.dmuon_plan_describe([(256, 512), (1000, 1500), (130, 70)], ns_backend="direct")
    assert all(m["form"] == "direct" for m in plan["matrices"])
    m = plan["matrices"]
    assert (m[1]["m_pad"], m[1]["n_pad"]) == (1024, 1536)
    assert (m[2]["m_pad"], m[2]["n_pad"]) == (128, 256) and m[2]["tall"]
    assert len(plan["launches"]) == 15
    assert all(l["sym_tasks"] + l["left_tasks"] == l["tasks"] for l in plan["launches"])
    p0 = dm.dmuon_plan_describe([(256, 512)], ns_steps=0)
    assert p0["launches"] == []


def test_plan_tile_choice(dm):
    import dmuon_inputs as di
    big = dm.dmuon_plan_describe([(m.rows, m.cols) for m in di.workload(2).matrices])
    assert big["tile"] == 256 and all(m["tile"] == 256 for m in big["matrices"])
    assert all(m["m_pad"] % 256 == 0 and m["n_pad"] % 256 == 0 for m in big["matrices"])
    # the 196 matrices still form one launch per stage and operand form
    assert len(big["launches"]) == 16 and big["launches"][0]["tasks"] == 196
    # one 3B layer: 410 such tiles, mostly of 3072-wide matrices
    layer = dm.dmuon_plan_describe([(m.rows, m.cols) for m in di.workload(1).matrices])
    assert layer["tile"] == 256
    # too few 256-tiles, or mostly narrow matrices: 128
    assert dm.dmuon_plan_describe([(3072, 8192)])["tile"] == 128
    assert dm.dmuon_plan_describe([(1024, 1024)] * 16)["tile"] == 128
    assert dm.dmuon_plan_describe([(4096, 4096)])["tile"] == 256
    # in a big batch, matrices narrower than 256 keep 128-tiles in launches of their own
    mixed = dm.dmuon_plan_describe([(m.rows, m.cols) for m in di.workload(2).matrices] + [(128, 2048)])
    assert mixed["matrices"][-1]["tile"] == 128 and mixed["matrices"][-1]["m_pad"] == 128
    assert {l["tile"] for l in mixed["launches"]} == {128, 256}
    assert dm.dmuon_plan_describe([(4096, 4096)], ns_precision="f32")["tile"] == 64
    # fp32 products: 128-tiles once the first stage has two waves of them;
    # matrices narrower than 128 keep 64-tiles in launches of their own
    w4 = [(m.rows, m.cols) for m in di.workload(4).matrices]
    p4 = dm.dmuon_plan_describe(w4, ns_precision="f32")
    assert p4["tile"] == 128 and all(m["tile"] == 128 for m in p4["matrices"])
    assert all(m["m_pad"] % 128 == 0 and m["n_pad"] % 128 == 0 for m in p4["matrices"])
    p4m = dm.dmuon_plan_describe(w4 + [(64, 300)], ns_precision="f32")
    assert p4m["matrices"][-1]["tile"] == 64 and {l["tile"] for l in p4m["launches"]} == {64, 128}


def _tile_from_info(info, shapes, prec):
    """The tile edge the rule stated by dmuon_backend_info picks for a batch."""
    if prec == "bf16":
        g = info["ns_gemm_bf16"]
        rule = g["big_tile_rule"]
        small, big = g["tiles"]
        tiles = wide = 0
        for r, c in shapes:
            t = -(-min(r, c) // big)
            tiles += t * (t + 1) // 2
            if min(r, c) >= rule["wide_min_dim"]:
                wide += t * (t + 1) // 2
        use_big = tiles >= rule["min_first_stage_tiles"] and wide >= rule["min_wide_share"] * tiles
    else:
        g = info["ns_gemm_f32"]
        rule = g["big_tile_rule"]
        small, big = g["tiles"]
        tiles = 0
        for r, c in shapes:
            t = -(-min(r, c) // big)
            tiles += t * (t + 1) // 2
        use_big = tiles >= rule["min_first_stage_tiles"]
    per_matrix = [big if use_big and min(r, c) >= rule["min_matrix_dim"] else small for r, c in shapes]
    return (big if use_big else small), per_matrix


def test_backend_info_describes_the_plan(dm, monkeypatch):
    """dmuon_backend_info states the kernels' tile edges and the rule that
    picks them; the planner's choice for every workload and precision is the
    one that rule gives."""
    import dmuon_inputs as di
    monkeypatch.delenv("DMUON_GEMM_TILE", raising=False)
    monkeypatch.delenv("DMUON_GEMM_TILE_F32", raising=False)
    info = dm.dmuon_backend_info()
    tiles = info["ns_gemm_bf16"]["tiles"]
    assert info["ns_gemm_bf16"]["mfma"] == {str(tiles[0]): "v_mfma_f32_32x32x16_bf16",
                                            str(tiles[1]): "v_mfma_f32_16x16x32_bf16"}
    assert info["ns_gemm_f32"]["mfma"] == "v_mfma_f32_32x32x2f32"
    batches = [[(m.rows, m.cols) for m in di.workload(k).matrices] for k in range(5)]
    batches += [[(3072, 8192)], [(1024, 1024)] * 16, [(4096, 4096)], [(128, 2048)] * 40,
                [(m.rows, m.cols) for m in di.workload(2).matrices] + [(128, 2048)]]
    for shapes in batches:
        for prec in ("bf16", "f32"):
            plan = dm.dmuon_plan_describe(shapes, ns_precision=prec)
            tile, per = _tile_from_info(info, shapes, prec)
            assert plan["tile"] == tile, (len(shapes), prec)
            assert [m["tile"] for m in plan["matrices"]] == per, (len(shapes), prec)
            assert {l["tile"] for l in plan["launches"]} <= set(info["ns_gemm_" + prec]["tiles"])
    env = info["tile_override_env"]
    assert (env["bf16"], env["f32"]) == ("DMUON_GEMM_TILE", "DMUON_GEMM_TILE_F32")


def test_stream_groups_for_small_batches(dm):
    """A bf16 batch whose first NS stage has fewer than 768 tiles of 256 runs
    as two groups balanced by m^2 n (the second on the library's own
    stream); larger batches, single matrices and fp32 products keep one."""
    import dmuon_inputs as di
    def groups(shapes, **hp):
        return dm.dmuon_plan_describe(shapes, **hp)["stream_groups"]
    def ns_cost(r, c, k=5):
        # flops of the planned products, symmetric ones counted once
        m, n = min(r, c), max(r, c)
        if n < 2 * m:                              # the gram backend's standard form
            return k * (3 * m * m * n + m ** 3)
        return 3 * m * m * n + (4 * k - 3) * m ** 3
    layer = [(m.rows, m.cols) for m in di.workload(1).matrices]
    g = groups(layer)
    assert len(g) == 2 and sorted(g[0] + g[1]) == list(range(7))
    cost = [ns_cost(r, c) for r, c in layer]
    loads = sorted(sum(cost[i] for i in grp) for grp in g)
    assert loads[1] - loads[0] <= max(cost)       # the greedy split's bound
    assert loads[1] <= 1.4 * loads[0]
    assert len(groups([(m.rows, m.cols) for m in di.workload(2).matrices])) == 1
    assert len(groups([(m.rows, m.cols) for m in di.workload(3).matrices])) == 1
    assert groups([(4096, 4096)]) == [[0]]
    assert len(groups(layer, ns_precision="f32")) == 1
    # equal matrices: an even count splits in halves; three (2:1) and five
    # (3:2) are too uneven and keep one stream
    assert groups([(3072, 8192)] * 4) == [[0, 2], [1, 3]]
    assert len(groups([(3072, 3072)] * 3)) == 1
    assert len(groups([(2048, 8192)] * 5)) == 1
    # the workspace of a split batch holds both groups' plans
    split_ws = dm.dmuon_orthogonalize_workspace_size(layer)
    whole = dm.dmuon_plan_describe(layer)["workspace_bytes"]
    assert split_ws >= whole * 0.9


def test_plan_tile_override(dm, monkeypatch):
    """DMUON_GEMM_TILE / DMUON_GEMM_TILE_F32 force the tile edge of their
    precision only."""
    monkeypatch.setenv("DMUON_GEMM_TILE", "256")
    monkeypatch.setenv("DMUON_GEMM_TILE_F32", "128")
    assert dm.dmuon_plan_describe([(300, 500)])["tile"] == 256
    p = dm.dmuon_plan_describe([(300, 500), (100, 700)], ns_precision="f32")
    assert p["tile"] == 128 and [m["tile"] for m in p["matrices"]] == [128, 64]
    monkeypatch.setenv("DMUON_GEMM_TILE_F32", "64")
    assert dm.dmuon_plan_describe([(m.rows, m.cols) for m in __import__("dmuon_inputs").workload(4).matrices],
                                  ns_precision="f32")["tile"] == 64
    monkeypatch.delenv("DMUON_GEMM_TILE")
    assert dm.dmuon_plan_describe([(300, 500)])["tile"] == 128


def test_tile_maps_cover_every_tile_once(dm):
    import dmuon_inputs as di
    cases = [[(m.rows, m.cols) for m in di.workload(k).matrices] for k in (1, 2, 4)]
    cases.append([(1000, 1500), (130, 70), (2048, 128), (64, 64), (1, 300)])
    for shapes in cases:
        for extra in ({}, {"ns_backend": "direct"}, {"ns_precision": "f32"}):
            plan = dm.dmuon_plan_describe(shapes, **extra)
            assert plan["tile_map_valid"] is True, (len(shapes), extra)
    # the element count must fit the 16-bit tile coordinates
    with pytest.raises(dm.DmuonError):
        dm.dmuon_plan_describe([(1 << 23, 16)])


def test_clip_argument_errors_before_launch(dm):
    """Every clipping argument check runs before anything touches a device
    (fake device addresses are never dereferenced)."""
    lib = dm._lib

    def grads(specs):
        arr = (dm.dmuon_grad_t * len(specs))()
        base = 1 << 41
        for i, (numel, dt, bucket) in enumerate(specs):
            arr[i].numel, arr[i].grad, arr[i].dtype, arr[i].bucket = numel, base + i * (1 << 30), dt, bucket
        return arr

    def call(g, n, nb=2, mx=(1.0, 1.0), p=2.0, ws=1 << 40, wsb=1 << 40):
        m = (ctypes.c_double * len(mx))(*mx)
        return lib.dmuon_clip_grad_norm(g, n, nb, m, p, None, ws, wsb, None)

    ok = grads([(1000, dm.DMUON_BF16, 0), (77, dm.DMUON_F32, 1)])
    need = lib.dmuon_clip_workspace_size(ok, 2, 2)
    # one 64 KB chunk per gradient here: 2 blocks of fp64 partials plus the tables
    assert 2 * 8 < need < 4096
    assert call(ok, -1) == dm.DMUON_ERR_INVALID_ARG
    assert call(ok, 2, nb=0) == dm.DMUON_ERR_INVALID_ARG
    assert call(grads([(1000, dm.DMUON_BF16, 2)]), 1) == dm.DMUON_ERR_INVALID_ARG       # bucket out of range
    assert call(grads([(0, dm.DMUON_BF16, 0)]), 1) == dm.DMUON_ERR_INVALID_ARG          # empty gradient
    assert call(grads([(10, 5, 0)]), 1) == dm.DMUON_ERR_UNSUPPORTED                     # dtype
    assert call(ok, 2, mx=(1.0, -1.0)) == dm.DMUON_ERR_INVALID_ARG                      # max_norm < 0
    assert call(ok, 2, mx=(float("nan"), 1.0)) == dm.DMUON_ERR_INVALID_ARG
    for p in (0.0, -2.0, float("nan")):
        assert call(ok, 2, p=p) == dm.DMUON_ERR_INVALID_ARG, p
    nul = grads([(1000, dm.DMUON_BF16, 0)])
    nul[0].grad = None
    assert call(nul, 1) == dm.DMUON_ERR_INVALID_ARG
    assert call(ok, 2, ws=None) == dm.DMUON_ERR_WORKSPACE
    assert call(ok, 2, wsb=need - 1) == dm.DMUON_ERR_WORKSPACE
    assert call(ok, 2, ws=(1 << 40) + 8, wsb=need) == dm.DMUON_ERR_INVALID_ARG          # misaligned
    dup = grads([(1000, dm.DMUON_BF16, 0), (1000, dm.DMUON_BF16, 1)])
    dup[1].grad = dup[0].grad + 100
    assert call(dup, 2) == dm.DMUON_ERR_ALIASING
    assert call(ok, 0, ws=None, wsb=0) == dm.DMUON_OK                                    # nothing to do


def test_clip_noalloc_errors_before_launch(dm):
    """The allocation-free clip checks its arguments, and that the gradients
    fit its fixed scratch, before it looks anything up on a device (the fake
    device addresses are never dereferenced)."""
    lib = dm._lib
    assert dm.DMUON_NOALLOC_SCRATCH_BYTES == 4 << 20

    def grads(specs):
        arr = (dm.dmuon_grad_t * len(specs))()
        base = 1 << 41
        for i, (numel, dt, bucket) in enumerate(specs):
            arr[i].numel, arr[i].grad, arr[i].dtype, arr[i].bucket = numel, base + i * (1 << 36), dt, bucket
        return arr

    def call(g, n, nb=1, mx=(1.0,), p=2.0):
        m = (ctypes.c_double * len(mx))(*mx)
        return lib.dmuon_clip_grad_norm_noalloc(g, n, nb, m, p, None, None)

    ok = grads([(1000, dm.DMUON_BF16, 0)])
    assert call(ok, -1) == dm.DMUON_ERR_INVALID_ARG
    assert call(ok, 1, nb=0) == dm.DMUON_ERR_INVALID_ARG
    assert call(ok, 1, p=0.0) == dm.DMUON_ERR_INVALID_ARG
    assert call(grads([(10, 5, 0)]), 1) == dm.DMUON_ERR_UNSUPPORTED
    assert call(ok, 0) == dm.DMUON_OK
    # the largest bf16 gradient (in 64 KB chunks) whose scratch fits, then one chunk more
    def need(chunks):
        return lib.dmuon_clip_workspace_size(grads([(chunks * 32768, dm.DMUON_BF16, 0)]), 1, 1)
    lo, hi = 1, 1 << 21
    while lo + 1 < hi:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if need(mid) <= dm.DMUON_NOALLOC_SCRATCH_BYTES else (lo, mid)
    assert need(lo) <= dm.DMUON_NOALLOC_SCRATCH_BYTES < need(lo + 1)
    assert lo * 65536 > 30 * 10**9            # about 30 GB of gradients in one bucket
    big = grads([((lo + 1) * 32768, dm.DMUON_BF16, 0)])
    assert call(big, 1) == dm.DMUON_ERR_WORKSPACE
    assert "scratch" in dm.dmuon_last_error()
    many = grads([(100, dm.DMUON_F32, 0)] * 140000)      # the gradient table alone is too large
    assert call(many, 140000) == dm.DMUON_ERR_WORKSPACE


def test_sharded_argument_errors_before_launch(dm):
    """Every argument check of the sharded entry point runs before anything
    touches a device (fake device addresses are never dereferenced)."""
    lib = dm._lib
    h, _keep = dm._hparams()

    def mats(specs, addr=1 << 42):
        """specs: list of (split, [(rows, cols), ...])"""
        shapes = [[rc for rc in sh] for _, sh in specs]
        arr, keep = dm._sharded(shapes, [sp for sp, _ in specs])
        for i, (_, sh) in enumerate(specs):
            for j in range(len(sh)):
                arr[i].shards[j].in_ = addr
                arr[i].shards[j].out = addr
                addr += 1 << 32
        return arr, keep

    def call(arr, n, ws=1 << 46, wsb=1 << 45, io=dm.DMUON_BF16):
        return lib.dmuon_orthogonalize_sharded(arr, n, io, ctypes.byref(h), ws, wsb, None)

    ok, k1 = mats([(1, [(256, 300), (256, 700)]), (0, [(100, 512), (412, 512)])])
    need = lib.dmuon_orthogonalize_sharded_workspace_size(ok, 2, ctypes.byref(h))
    assert need > 0
    # one shard costs what the unsharded call costs, apart from the table
    one, k2 = mats([(1, [(256, 1000)])])
    rows, cols = (ctypes.c_int64 * 1)(256), (ctypes.c_int64 * 1)(1000)
    assert abs(lib.dmuon_orthogonalize_sharded_workspace_size(one, 1, ctypes.byref(h)) -
               lib.dmuon_orthogonalize_workspace_size(rows, cols, 1, ctypes.byref(h))) < 4096
    assert call(ok, -1) == dm.DMUON_ERR_INVALID_ARG
    bad, k3 = mats([(1, [(256, 300), (255, 700)])])          # d differs
    assert call(bad, 1) == dm.DMUON_ERR_INVALID_ARG
    assert "unsplit" in dm.dmuon_last_error()
    bad, k4 = mats([(2, [(256, 300)])])                       # split
    assert call(bad, 1) == dm.DMUON_ERR_INVALID_ARG
    bad, k5 = mats([(1, [(256, 300)])])
    bad[0].nshards = 0
    assert call(bad, 1) == dm.DMUON_ERR_INVALID_ARG
    bad, k6 = mats([(1, [(0, 300)])])
    assert call(bad, 1) == dm.DMUON_ERR_INVALID_ARG
    assert call(ok, 2, io=7) == dm.DMUON_ERR_UNSUPPORTED
    assert call(ok, 2, wsb=16) == dm.DMUON_ERR_WORKSPACE
    assert call(ok, 2, ws=(1 << 46) + 8) == dm.DMUON_ERR_INVALID_ARG        # alignment
    nul, k7 = mats([(1, [(256, 300)])])
    nul[0].shards[0].out = None
    assert call(nul, 1) == dm.DMUON_ERR_INVALID_ARG
    dup, k8 = mats([(1, [(256, 300), (256, 700)])])
    dup[0].shards[1].out = dup[0].shards[0].out
    assert call(dup, 1) == dm.DMUON_ERR_ALIASING
    assert call(ok, 0) == dm.DMUON_OK


def test_adamw_argument_errors_before_launch(dm):
    """Every AdamW argument check runs before anything touches a device."""
    lib = dm._lib
    base = 1 << 43

    def tensors(specs):
        arr = (dm.dmuon_adamw_tensor_t * len(specs))()
        for i, (numel, pdt, gdt, group) in enumerate(specs):
            a = base + i * (1 << 34)
            arr[i].numel, arr[i].param, arr[i].grad = numel, a, a + (1 << 32)
            arr[i].exp_avg, arr[i].exp_avg_sq = a + (2 << 32), a + (3 << 32)
            arr[i].param_dtype, arr[i].grad_dtype, arr[i].group = pdt, gdt, group
        return arr

    def groups(specs):
        arr = (dm.dmuon_adamw_group_t * len(specs))()
        for i, (lr, b1, b2, eps, wd, step) in enumerate(specs):
            arr[i].lr, arr[i].beta1, arr[i].beta2, arr[i].eps, arr[i].weight_decay, arr[i].step = \
                lr, b1, b2, eps, wd, step
        return arr

    good_g = groups([(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)])

    def call(t, n, g=good_g, ng=1, ws=1 << 47, wsb=1 << 20):
        return lib.dmuon_adamw_step(t, n, g, ng, ws, wsb, None)

    ok = tensors([(1000, dm.DMUON_BF16, dm.DMUON_BF16, 0), (77, dm.DMUON_F32, dm.DMUON_F32, 0)])
    assert dm.dmuon_adamw_workspace_size(2) >= 2 * 64 and dm.dmuon_adamw_workspace_size(0) == 0
    assert call(ok, -1) == dm.DMUON_ERR_INVALID_ARG
    assert call(ok, 0) == dm.DMUON_OK
    assert call(ok, 2, ng=0) == dm.DMUON_ERR_INVALID_ARG
    for bad in ((float("nan"), 0.9, 0.999, 1e-8, 0.01, 1), (1e-3, 1.0, 0.999, 1e-8, 0.01, 1),
                (1e-3, 0.9, -0.1, 1e-8, 0.01, 1), (1e-3, 0.9, 0.999, -1.0, 0.01, 1),
                (1e-3, 0.9, 0.999, 1e-8, float("inf"), 1), (1e-3, 0.9, 0.999, 1e-8, 0.01, 0)):
        assert call(ok, 2, g=groups([bad])) == dm.DMUON_ERR_INVALID_ARG, bad
    assert call(tensors([(0, 1, 1, 0)]), 1) == dm.DMUON_ERR_INVALID_ARG
    assert call(tensors([(10, 1, 1, 1)]), 1) == dm.DMUON_ERR_INVALID_ARG          # group index
    assert call(tensors([(10, 5, 1, 0)]), 1) == dm.DMUON_ERR_UNSUPPORTED
    nul = tensors([(10, 1, 1, 0)])
    nul[0].exp_avg = None
    assert call(nul, 1) == dm.DMUON_ERR_INVALID_ARG
    ali = tensors([(10, 1, 1, 0), (10, 1, 1, 0)])
    ali[1].exp_avg_sq = ali[0].param
    assert call(ali, 2) == dm.DMUON_ERR_ALIASING
    assert call(ok, 2, wsb=16) == dm.DMUON_ERR_WORKSPACE
    assert call(ok, 2, ws=(1 << 47) + 8) == dm.DMUON_ERR_INVALID_ARG
    skip = tensors([(10, 1, 1, 0)])
    skip[0].grad = None
    assert call(skip, 1, ws=None, wsb=0) == dm.DMUON_OK                             # nothing to do


def test_fused_clip_entry_points_reject_null(dm):
    lib = dm._lib
    h, _keep = dm._hparams()
    mats = _mats(dm, [(256, 512)])
    assert lib.dmuon_step_scaled(mats, 1, ctypes.byref(h), None, 1 << 40, 1 << 40, None) == dm.DMUON_ERR_INVALID_ARG
    assert "grad_scale" in dm.dmuon_last_error()
    arr = (dm.dmuon_grad_t * 1)()
    arr[0].numel, arr[0].grad, arr[0].dtype, arr[0].bucket = 100, 1 << 41, dm.DMUON_BF16, 0
    mx = (ctypes.c_double * 1)(1.0)
    assert lib.dmuon_clip_coefficients(arr, 1, 1, mx, 2.0, None, None, 1 << 42, 1 << 20, None) == \
        dm.DMUON_ERR_INVALID_ARG
    assert "coef_out" in dm.dmuon_last_error()


def test_bench_power_sampler_without_a_gpu():
    """The benchmark's board-power sampler reports None, and does not raise,
    where amdsmi or a GPU is not available (as in this container)."""
    import time
    import bench
    p = bench.PowerSampler()
    p.start()
    time.sleep(0.1)
    summary = p.stop()
    if p.handle is None:
        assert summary is None
    else:       # a box with a GPU: the summary carries the readings
        assert summary is None or {"socket_w_median", "cap_w", "gfxclk_mhz_median"} <= set(summary)
