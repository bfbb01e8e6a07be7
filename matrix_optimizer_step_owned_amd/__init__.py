"""Python binding of the dmuon C ABI (include/dmuon.h): argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors
are PyTorch tensors (device memory and streams come from PyTorch); all the
arithmetic of the step runs in the library's HIP kernels.  The library must
have been built (``__graft_entry__.build()`` or ``python
matrix_optimizer_step_owned_amd/_build.py``); importing this package without it
raises ImportError.
"""
from __future__ import annotations

import ctypes
import json
import os
from typing import List, Optional, Sequence, Tuple

import torch  # loaded first so that the library binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdmuon.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")

_lib = ctypes.CDLL(LIB_PATH)

DMUON_OK = 0
DMUON_ERR_INVALID_ARG = -1
DMUON_ERR_UNSUPPORTED = -2
DMUON_ERR_WORKSPACE = -3
DMUON_ERR_ALIASING = -4
DMUON_ERR_HIP = -5

DMUON_F32 = 0
DMUON_BF16 = 1
DMUON_NS_GRAM = 0
DMUON_NS_DIRECT = 1
DMUON_NS_PREC_BF16 = 0
DMUON_NS_PREC_F32 = 1

_BACKENDS = {"gram": DMUON_NS_GRAM, "direct": DMUON_NS_DIRECT}
_PRECISIONS = {"bf16": DMUON_NS_PREC_BF16, "f32": DMUON_NS_PREC_F32}
_DTYPES = {torch.float32: DMUON_F32, torch.bfloat16: DMUON_BF16}


class dmuon_matrix_t(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("momentum", ctypes.c_void_p),
                ("param_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32)]


class dmuon_hparams_t(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("momentum", ctypes.c_double),
                ("nesterov", ctypes.c_int32), ("ns_steps", ctypes.c_int32),
                ("weight_decay", ctypes.c_double),
                ("ns_backend", ctypes.c_int32), ("ns_precision", ctypes.c_int32),
                ("ns_coeffs", ctypes.POINTER(ctypes.c_double)),
                ("ns_coeffs_len", ctypes.c_int32), ("eps", ctypes.c_double)]


class dmuon_grad_t(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("grad", ctypes.c_void_p),
                ("dtype", ctypes.c_int32), ("bucket", ctypes.c_int32)]


class dmuon_shard_t(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("in_", ctypes.c_void_p), ("out", ctypes.c_void_p)]


class dmuon_sharded_t(ctypes.Structure):
    _fields_ = [("shards", ctypes.POINTER(dmuon_shard_t)), ("nshards", ctypes.c_int32),
                ("split", ctypes.c_int32)]


class dmuon_adamw_group_t(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64)]


class dmuon_adamw_tensor_t(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("param_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
                ("group", ctypes.c_int32), ("pad_", ctypes.c_int32)]


_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)
_I64P = ctypes.POINTER(ctypes.c_int64)
_MP = ctypes.POINTER(dmuon_matrix_t)
_HP = ctypes.POINTER(dmuon_hparams_t)

EXPORTS = {
    "dmuon_hparams_default": (None, [_HP]),
    "dmuon_step_workspace_size": (ctypes.c_size_t, [_MP, ctypes.c_int32, _HP]),
    "dmuon_step": (ctypes.c_int, [_MP, ctypes.c_int32, _HP, _P, ctypes.c_size_t, _P]),
    "dmuon_step_scaled": (ctypes.c_int, [_MP, ctypes.c_int32, _HP, _PP, _P, ctypes.c_size_t, _P]),
    "dmuon_momentum_workspace_size": (ctypes.c_size_t, [_MP, ctypes.c_int32]),
    "dmuon_momentum": (ctypes.c_int, [_MP, ctypes.c_int32, _HP, _PP, ctypes.c_int32, _P, _P,
                                      ctypes.c_size_t, _P]),
    "dmuon_orthogonalize_workspace_size": (ctypes.c_size_t, [_I64P, _I64P, ctypes.c_int32, _HP]),
    "dmuon_orthogonalize": (ctypes.c_int, [_PP, _PP, _I64P, _I64P, ctypes.c_int32, ctypes.c_int32,
                                           _HP, _P, ctypes.c_size_t, _P]),
    "dmuon_orthogonalize_sharded_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(dmuon_sharded_t),
                                                                      ctypes.c_int32, _HP]),
    "dmuon_orthogonalize_sharded": (ctypes.c_int, [ctypes.POINTER(dmuon_sharded_t), ctypes.c_int32,
                                                   ctypes.c_int32, _HP, _P, ctypes.c_size_t, _P]),
    "dmuon_apply_update_workspace_size": (ctypes.c_size_t, [ctypes.c_int32]),
    "dmuon_apply_update": (ctypes.c_int, [_MP, ctypes.c_int32, _PP, ctypes.c_int32, _HP, _P,
                                          ctypes.c_size_t, _P]),
    "dmuon_clip_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(dmuon_grad_t), ctypes.c_int32,
                                                     ctypes.c_int32]),
    "dmuon_clip_grad_norm": (ctypes.c_int, [ctypes.POINTER(dmuon_grad_t), ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_double), ctypes.c_double, _P, _P,
                                            ctypes.c_size_t, _P]),
    "dmuon_clip_grad_norm_noalloc": (ctypes.c_int, [ctypes.POINTER(dmuon_grad_t), ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.POINTER(ctypes.c_double), ctypes.c_double, _P, _P]),
    "dmuon_clip_coefficients": (ctypes.c_int, [ctypes.POINTER(dmuon_grad_t), ctypes.c_int32, ctypes.c_int32,
                                               ctypes.POINTER(ctypes.c_double), ctypes.c_double, _P, _P, _P,
                                               ctypes.c_size_t, _P]),
    "dmuon_adamw_workspace_size": (ctypes.c_size_t, [ctypes.c_int32]),
    "dmuon_adamw_step": (ctypes.c_int, [ctypes.POINTER(dmuon_adamw_tensor_t), ctypes.c_int32,
                                        ctypes.POINTER(dmuon_adamw_group_t), ctypes.c_int32, _P, ctypes.c_size_t,
                                        _P]),
    "dmuon_assign_owners": (ctypes.c_int, [_I64P, _I64P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _HP,
                                           ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
    "dmuon_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dmuon_last_error": (ctypes.c_char_p, []),
    "dmuon_backend_info": (ctypes.c_char_p, []),
    "dmuon_plan_describe": (ctypes.c_int64, [_I64P, _I64P, ctypes.c_int32, _HP, ctypes.c_char_p,
                                             ctypes.c_size_t]),
    "dmuon_profile_begin": (ctypes.c_int, []),
    "dmuon_profile_end": (ctypes.c_int64, [ctypes.c_char_p, ctypes.c_size_t]),
}

for _name, (_res, _args) in EXPORTS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class DmuonError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _lib.dmuon_last_error().decode()
        super().__init__(f"{where}: {_lib.dmuon_status_string(status).decode()} ({status}): {detail}")


def _check(status: int, where: str) -> None:
    if status != DMUON_OK:
        raise DmuonError(status, where)


def dmuon_status_string(status: int) -> str:
    return _lib.dmuon_status_string(status).decode()


def dmuon_last_error() -> str:
    return _lib.dmuon_last_error().decode()


def dmuon_backend_info() -> dict:
    return json.loads(_lib.dmuon_backend_info().decode())


def dmuon_hparams_default() -> dict:
    hp = dmuon_hparams_t()
    _lib.dmuon_hparams_default(ctypes.byref(hp))
    return dict(lr=hp.lr, momentum=hp.momentum, nesterov=bool(hp.nesterov), ns_steps=hp.ns_steps,
                weight_decay=hp.weight_decay,
                ns_backend={v: k for k, v in _BACKENDS.items()}[hp.ns_backend],
                ns_precision={v: k for k, v in _PRECISIONS.items()}[hp.ns_precision],
                ns_coeffs=None, eps=hp.eps)


def _hparams(lr=0.02, momentum=0.95, nesterov=True, ns_steps=5, weight_decay=0.0,
             ns_backend="gram", ns_precision="bf16", ns_coeffs=None, eps=1e-7):
    hp = dmuon_hparams_t()
    hp.lr = float(lr)
    hp.momentum = float(momentum)
    hp.nesterov = 1 if nesterov else 0
    hp.ns_steps = int(ns_steps)
    hp.weight_decay = float(weight_decay)
    hp.ns_backend = _BACKENDS[ns_backend] if isinstance(ns_backend, str) else int(ns_backend)
    hp.ns_precision = _PRECISIONS[ns_precision] if isinstance(ns_precision, str) else int(ns_precision)
    keep = None
    if ns_coeffs is not None:
        flat = [float(v) for row in ns_coeffs for v in (row if hasattr(row, "__len__") else [row])]
        keep = (ctypes.c_double * len(flat))(*flat)
        hp.ns_coeffs = ctypes.cast(keep, ctypes.POINTER(ctypes.c_double))
        hp.ns_coeffs_len = len(flat)
    hp.eps = float(eps)
    return hp, keep


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _mat(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _matrices(params, grads, momenta) -> ctypes.Array:
    n = len(params)
    arr = (dmuon_matrix_t * max(n, 1))()
    for i in range(n):
        p = _mat(params[i], f"params[{i}]")
        m = arr[i]
        m.rows, m.cols = p.shape
        m.param = p.data_ptr()
        m.param_dtype = _dtype(p)
        g = grads[i] if grads is not None else None
        if g is not None:
            _mat(g, f"grads[{i}]")
            if tuple(g.shape) != tuple(p.shape):
                raise ValueError(f"grads[{i}] shape {tuple(g.shape)} != param shape {tuple(p.shape)}")
            m.grad = g.data_ptr()
            m.grad_dtype = _dtype(g)
        else:
            m.grad = None
            m.grad_dtype = m.param_dtype
        if momenta is not None and momenta[i] is not None:
            b = _mat(momenta[i], f"momenta[{i}]")
            if b.dtype != torch.float32 or tuple(b.shape) != tuple(p.shape):
                raise ValueError(f"momenta[{i}] must be float32 of the param's shape")
            m.momentum = b.data_ptr()
        else:
            m.momentum = None
    return arr


def _torch_stream(stream, device):
    """The stream the library's kernels go to, as a torch stream: the
    current stream by default, a torch stream as given, or a raw HIP stream
    handle wrapped as an external stream."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _stream(stream, device) -> int:
    return _torch_stream(stream, device).cuda_stream


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor], stream=None):
    """The caller's workspace, or one allocated here.  An allocated one
    belongs to the stream the kernels run on (so PyTorch's caching allocator
    hands its bytes to nothing else until that stream has passed the
    kernels that use them), whichever stream is current."""
    if nbytes == 0:
        return None, 0
    if workspace is None:
        ts = _torch_stream(stream, device)
        with torch.cuda.stream(ts):
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace, workspace.numel() * workspace.element_size()


def _ptrs(ts: Sequence[Optional[torch.Tensor]]):
    arr = (ctypes.c_void_p * max(len(ts), 1))()
    for i, t in enumerate(ts):
        arr[i] = t.data_ptr() if t is not None else None
    return arr


def dmuon_step_workspace_size(params, grads, momenta=None, **hp) -> int:
    mats = _matrices(params, grads, momenta)
    h, _k = _hparams(**hp)
    return int(_lib.dmuon_step_workspace_size(mats, len(params), ctypes.byref(h)))


def dmuon_step(params: List[torch.Tensor], grads: List[Optional[torch.Tensor]],
               momenta: List[torch.Tensor], *, workspace: Optional[torch.Tensor] = None,
               stream=None, grad_scale: Optional[torch.Tensor] = None,
               grad_scale_index: Optional[Sequence[int]] = None, **hp) -> None:
    """One Muon step over a batch of owned matrices (in place on params and
    momenta).  With ``grad_scale`` (a float64 device tensor of clipping
    coefficients, e.g. from dmuon_clip_coefficients) matrix i's gradient is
    scaled by grad_scale[grad_scale_index[i]] as it is read
    (dmuon_step_scaled); an index of -1 leaves that matrix unscaled."""
    n = len(params)
    if n == 0:
        return
    mats = _matrices(params, grads, momenta)
    h, _keep = _hparams(**hp)
    nbytes = int(_lib.dmuon_step_workspace_size(mats, n, ctypes.byref(h)))
    ws, wsb = _workspace(nbytes, params[0].device, workspace, stream)
    wsp = ws.data_ptr() if ws is not None else None
    st = _stream(stream, params[0].device)
    if grad_scale is None:
        _check(_lib.dmuon_step(mats, n, ctypes.byref(h), wsp, wsb, st), "dmuon_step")
        return
    if grad_scale.dtype != torch.float64 or not grad_scale.is_contiguous():
        raise TypeError("grad_scale must be a contiguous float64 tensor")
    idx = list(grad_scale_index) if grad_scale_index is not None else [0] * n
    if len(idx) != n or any(k >= grad_scale.numel() for k in idx):
        raise ValueError("grad_scale_index must give one index into grad_scale per matrix")
    base = grad_scale.data_ptr()
    ptrs = (ctypes.c_void_p * n)(*[base + 8 * int(k) if k >= 0 else None for k in idx])
    _check(_lib.dmuon_step_scaled(mats, n, ctypes.byref(h), ptrs, wsp, wsb, st), "dmuon_step_scaled")


def dmuon_momentum_workspace_size(grads, momenta) -> int:
    mats = _matrices(momenta, grads, momenta)
    return int(_lib.dmuon_momentum_workspace_size(mats, len(grads)))


def dmuon_momentum(grads: List[torch.Tensor], momenta: List[torch.Tensor],
                   ns_inputs: List[torch.Tensor], sumsq: torch.Tensor, *, momentum: float = 0.95,
                   nesterov: bool = True, workspace: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """Momentum stage: updates momenta, writes the wide-orientation NS inputs and sum(U^2)."""
    n = len(grads)
    if n == 0:
        return
    # the momentum buffers stand in for the (unused) params in the matrix records
    mats = _matrices(momenta, grads, momenta)
    dt = _dtype(ns_inputs[0])
    for i, u in enumerate(ns_inputs):
        r, c = grads[i].shape
        if tuple(u.shape) != (min(r, c), max(r, c)) or _dtype(u) != dt or not u.is_contiguous():
            raise ValueError(f"ns_inputs[{i}] must be a contiguous {min(r, c)}x{max(r, c)} tensor of one dtype")
    if sumsq.dtype != torch.float64 or sumsq.numel() < n:
        raise ValueError("sumsq must be a float64 tensor of n entries")
    h, _keep = _hparams(momentum=momentum, nesterov=nesterov)
    nbytes = int(_lib.dmuon_momentum_workspace_size(mats, n))
    ws, wsb = _workspace(nbytes, grads[0].device, workspace, stream)
    _check(_lib.dmuon_momentum(mats, n, ctypes.byref(h), _ptrs(ns_inputs), dt, sumsq.data_ptr(),
                               ws.data_ptr() if ws is not None else None, wsb,
                               _stream(stream, grads[0].device)), "dmuon_momentum")


def dmuon_orthogonalize_workspace_size(shapes: Sequence[Sequence[int]], **hp) -> int:
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[int(s[0]) for s in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[int(s[1]) for s in shapes])
    h, _k = _hparams(**hp)
    return int(_lib.dmuon_orthogonalize_workspace_size(rows, cols, n, ctypes.byref(h)))


def dmuon_orthogonalize(inputs: List[torch.Tensor], outputs: List[torch.Tensor], *,
                        workspace: Optional[torch.Tensor] = None, stream=None, **hp) -> None:
    """outputs[i] = NS(inputs[i]) (same shape and dtype as the input)."""
    n = len(inputs)
    if n == 0:
        return
    dt = _dtype(inputs[0])
    for i in range(n):
        _mat(inputs[i], f"inputs[{i}]")
        _mat(outputs[i], f"outputs[{i}]")
        if _dtype(inputs[i]) != dt or _dtype(outputs[i]) != dt or inputs[i].shape != outputs[i].shape:
            raise ValueError(f"inputs[{i}] / outputs[{i}] must share one shape and dtype")
    rows = (ctypes.c_int64 * n)(*[int(t.shape[0]) for t in inputs])
    cols = (ctypes.c_int64 * n)(*[int(t.shape[1]) for t in inputs])
    h, _keep = _hparams(**hp)
    nbytes = int(_lib.dmuon_orthogonalize_workspace_size(rows, cols, n, ctypes.byref(h)))
    ws, wsb = _workspace(nbytes, inputs[0].device, workspace, stream)
    _check(_lib.dmuon_orthogonalize(_ptrs(inputs), _ptrs(outputs), rows, cols, n, dt, ctypes.byref(h),
                                    ws.data_ptr() if ws is not None else None, wsb,
                                    _stream(stream, inputs[0].device)), "dmuon_orthogonalize")


def _sharded(shards: Sequence[Sequence[Tuple[int, int]]], splits: Sequence[int],
             ins=None, outs=None):
    """ctypes descriptors of sharded matrices (shapes, and device pointers
    when tensors are given); returns (array, objects to keep alive)."""
    n = len(shards)
    arr = (dmuon_sharded_t * max(n, 1))()
    keep = []
    for i, mat in enumerate(shards):
        sh = (dmuon_shard_t * max(len(mat), 1))()
        for j, (r, c) in enumerate(mat):
            sh[j].rows, sh[j].cols = int(r), int(c)
            if ins is not None:
                sh[j].in_ = ins[i][j].data_ptr()
                sh[j].out = outs[i][j].data_ptr()
        keep.append(sh)
        arr[i].shards = ctypes.cast(sh, ctypes.POINTER(dmuon_shard_t))
        arr[i].nshards = len(mat)
        arr[i].split = int(splits[i])
    return arr, keep


def _splits(split, n: int) -> List[int]:
    return [int(split)] * n if isinstance(split, int) else [int(v) for v in split]


def dmuon_orthogonalize_sharded_workspace_size(shards: Sequence[Sequence[Sequence[int]]], split=1,
                                               **hp) -> int:
    """Workspace bytes of dmuon_orthogonalize_sharded for these shard shapes."""
    arr, _k1 = _sharded(shards, _splits(split, len(shards)))
    h, _k2 = _hparams(**hp)
    return int(_lib.dmuon_orthogonalize_sharded_workspace_size(arr, len(shards), ctypes.byref(h)))


def dmuon_orthogonalize_sharded(inputs: List[List[torch.Tensor]], outputs: List[List[torch.Tensor]],
                                split=1, *, workspace: Optional[torch.Tensor] = None, stream=None,
                                **hp) -> None:
    """outputs[i][s] = shard s of NS(U_i), where U_i is the matrix whose
    column blocks (split = 1) or row blocks (split = 0) are inputs[i]
    (``split`` one value or one per matrix); the Gram matrices of the shards
    are summed, the shards themselves are never joined."""
    n = len(inputs)
    if n == 0:
        return
    dt = _dtype(inputs[0][0])
    for i in range(n):
        if len(outputs[i]) != len(inputs[i]):
            raise ValueError(f"outputs[{i}] must have one tensor per shard")
        for j, (a, b) in enumerate(zip(inputs[i], outputs[i])):
            _mat(a, f"inputs[{i}][{j}]")
            _mat(b, f"outputs[{i}][{j}]")
            if _dtype(a) != dt or _dtype(b) != dt or a.shape != b.shape:
                raise ValueError(f"inputs[{i}][{j}] / outputs[{i}][{j}] must share one shape and dtype")
    shapes = [[tuple(t.shape) for t in mat] for mat in inputs]
    arr, _keep = _sharded(shapes, _splits(split, n), inputs, outputs)
    h, _keep2 = _hparams(**hp)
    nbytes = int(_lib.dmuon_orthogonalize_sharded_workspace_size(arr, n, ctypes.byref(h)))
    dev = inputs[0][0].device
    ws, wsb = _workspace(nbytes, dev, workspace, stream)
    _check(_lib.dmuon_orthogonalize_sharded(arr, n, dt, ctypes.byref(h),
                                            ws.data_ptr() if ws is not None else None, wsb,
                                            _stream(stream, dev)), "dmuon_orthogonalize_sharded")


def dmuon_adamw_workspace_size(n: int) -> int:
    return int(_lib.dmuon_adamw_workspace_size(int(n)))


def dmuon_adamw_step(params: List[torch.Tensor], grads: List[Optional[torch.Tensor]], exp_avgs: List[torch.Tensor],
                     exp_avg_sqs: List[torch.Tensor], *, step: int, lr: float = 1e-3, betas=(0.9, 0.999),
                     eps: float = 1e-8, weight_decay: float = 0.01, groups: Optional[Sequence[dict]] = None,
                     group_index: Optional[Sequence[int]] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    """One fused AdamW step over every tensor (in place).  One hyperparameter
    set from the keywords, or ``groups`` (dicts with lr, betas, eps,
    weight_decay, step) with ``group_index`` naming each tensor's group."""
    n = len(params)
    if n == 0:
        return
    if groups is None:
        groups = [dict(lr=lr, betas=betas, eps=eps, weight_decay=weight_decay, step=step)]
        group_index = [0] * n
    if group_index is None or len(group_index) != n:
        raise ValueError("group_index must name one group per tensor")
    ga = (dmuon_adamw_group_t * len(groups))()
    for k, g in enumerate(groups):
        b1, b2 = g.get("betas", (0.9, 0.999))
        ga[k].lr, ga[k].beta1, ga[k].beta2 = float(g.get("lr", 1e-3)), float(b1), float(b2)
        ga[k].eps, ga[k].weight_decay = float(g.get("eps", 1e-8)), float(g.get("weight_decay", 0.01))
        ga[k].step = int(g["step"])
    ta = (dmuon_adamw_tensor_t * n)()
    for i in range(n):
        p, gr, m, v = params[i], grads[i], exp_avgs[i], exp_avg_sqs[i]
        for t, what in ((p, "params"), (m, "exp_avgs"), (v, "exp_avg_sqs")):
            if not t.is_contiguous():
                raise ValueError(f"{what}[{i}] must be contiguous")
        if m.dtype != torch.float32 or v.dtype != torch.float32:
            raise TypeError("exp_avg and exp_avg_sq must be float32")
        if m.numel() != p.numel() or v.numel() != p.numel() or (gr is not None and gr.numel() != p.numel()):
            raise ValueError(f"tensors[{i}]: sizes differ")
        ta[i].numel = p.numel()
        ta[i].param = p.data_ptr()
        ta[i].grad = gr.data_ptr() if gr is not None else None
        ta[i].exp_avg = m.data_ptr()
        ta[i].exp_avg_sq = v.data_ptr()
        ta[i].param_dtype = _dtype(p)
        ta[i].grad_dtype = _dtype(gr) if gr is not None else _dtype(p)
        ta[i].group = int(group_index[i])
        if gr is not None and not gr.is_contiguous():
            raise ValueError(f"grads[{i}] must be contiguous")
    ws, wsb = _workspace(dmuon_adamw_workspace_size(n), params[0].device, workspace, stream)
    _check(_lib.dmuon_adamw_step(ta, n, ga, len(groups), ws.data_ptr() if ws is not None else None, wsb,
                                 _stream(stream, params[0].device)), "dmuon_adamw_step")


DMUON_COST_NUMEL = 0
DMUON_COST_NS_NOMINAL = 1
DMUON_COST_ROOFLINE = 2
_COST_MODELS = {"numel": DMUON_COST_NUMEL, "ns_nominal": DMUON_COST_NS_NOMINAL, "roofline": DMUON_COST_ROOFLINE}


def dmuon_assign_owners(shapes: Sequence[Sequence[int]], nranks: int, cost_model: str = "ns_nominal",
                        **hp) -> dict:
    """Owner rank of every matrix: {"owner", "cost", "loads", "imbalance"}."""
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[int(s[0]) for s in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[int(s[1]) for s in shapes])
    owner = (ctypes.c_int32 * max(n, 1))()
    cost = (ctypes.c_double * max(n, 1))()
    loads = (ctypes.c_double * max(int(nranks), 1))()
    imb = ctypes.c_double()
    h, _keep = _hparams(**hp)
    model = _COST_MODELS[cost_model] if isinstance(cost_model, str) else int(cost_model)
    _check(_lib.dmuon_assign_owners(rows, cols, n, int(nranks), model, ctypes.byref(h), owner, cost, loads,
                                    ctypes.byref(imb)), "dmuon_assign_owners")
    return {"owner": list(owner)[:n], "cost": list(cost)[:n], "loads": list(loads)[:int(nranks)],
            "imbalance": imb.value}


def dmuon_apply_update(params: List[torch.Tensor], updates: List[torch.Tensor], *, lr: float = 0.02,
                       weight_decay: float = 0.0, workspace: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    """W <- W*(1 - lr*wd) - lr*0.2*sqrt(max(m,n))*O for every matrix (in place)."""
    n = len(params)
    if n == 0:
        return
    mats = _matrices(params, None, None)
    dt = _dtype(updates[0])
    for i, u in enumerate(updates):
        _mat(u, f"updates[{i}]")
        if u.shape != params[i].shape or _dtype(u) != dt:
            raise ValueError(f"updates[{i}] must have the param's shape and one dtype")
    h, _keep = _hparams(lr=lr, weight_decay=weight_decay)
    nbytes = int(_lib.dmuon_apply_update_workspace_size(n))
    ws, wsb = _workspace(nbytes, params[0].device, workspace, stream)
    _check(_lib.dmuon_apply_update(mats, n, _ptrs(updates), dt, ctypes.byref(h),
                                   ws.data_ptr() if ws is not None else None, wsb,
                                   _stream(stream, params[0].device)), "dmuon_apply_update")


def dmuon_clip_grad_norm(grads: List[torch.Tensor], max_norm, *, norm_type: float = 2.0,
                         buckets: Optional[Sequence[int]] = None, total_norm: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Clip gradients in place by their global p-norm, per bucket (every
    gradient in bucket 0 unless ``buckets`` is given; ``max_norm`` a number or
    one per bucket).  Returns the per-bucket totals (float64, on the device)."""
    n = len(grads)
    if buckets is None:
        buckets = [0] * n
    if len(buckets) != n:
        raise ValueError("buckets must have one entry per gradient")
    nb = (max(buckets) + 1) if n else 1
    if isinstance(max_norm, (int, float)):
        max_norm = [float(max_norm)] * nb
    nb = max(nb, len(max_norm))
    if len(max_norm) != nb:
        raise ValueError("max_norm must have one value per bucket")
    arr = (dmuon_grad_t * max(n, 1))()
    for i, g in enumerate(grads):
        if not g.is_contiguous():
            raise ValueError(f"grads[{i}] must be contiguous")
        arr[i].numel = g.numel()
        arr[i].grad = g.data_ptr()
        arr[i].dtype = _dtype(g)
        arr[i].bucket = int(buckets[i])
    if n == 0:
        return torch.zeros(nb, dtype=torch.float64)
    device = grads[0].device
    if total_norm is None:
        with torch.cuda.stream(_torch_stream(stream, device)):
            total_norm = torch.empty(nb, dtype=torch.float64, device=device)
    mx = (ctypes.c_double * nb)(*[float(v) for v in max_norm])
    nbytes = int(_lib.dmuon_clip_workspace_size(arr, n, nb)) if n else 0
    ws, wsb = _workspace(nbytes, device, workspace, stream)
    _check(_lib.dmuon_clip_grad_norm(arr, n, nb, mx, float(norm_type), total_norm.data_ptr(),
                                     ws.data_ptr() if ws is not None else None, wsb, _stream(stream, device)),
           "dmuon_clip_grad_norm")
    return total_norm


DMUON_NOALLOC_SCRATCH_BYTES = 4 << 20


def _grad_descs(grads, buckets):
    arr = (dmuon_grad_t * max(len(grads), 1))()
    for i, g in enumerate(grads):
        if not g.is_contiguous():
            raise ValueError(f"grads[{i}] must be contiguous")
        arr[i].numel, arr[i].grad, arr[i].dtype, arr[i].bucket = g.numel(), g.data_ptr(), _dtype(g), int(buckets[i])
    return arr


def dmuon_clip_grad_norm_noalloc(grads: List[torch.Tensor], max_norm, *, norm_type: float = 2.0,
                                 buckets: Optional[Sequence[int]] = None,
                                 total_norm: Optional[torch.Tensor] = None, stream=None) -> Optional[torch.Tensor]:
    """dmuon_clip_grad_norm without a workspace and without any allocation:
    the library's per-GPU scratch array holds the clip's scratch.  The
    per-bucket totals go to ``total_norm`` (a float64 device tensor of one
    entry per bucket) if given, and are returned; nothing is allocated
    here either."""
    n = len(grads)
    if buckets is None:
        buckets = [0] * n
    if len(buckets) != n:
        raise ValueError("buckets must have one entry per gradient")
    nb = (max(buckets) + 1) if n else 1
    if isinstance(max_norm, (int, float)):
        max_norm = [float(max_norm)] * nb
    nb = max(nb, len(max_norm))
    if len(max_norm) != nb:
        raise ValueError("max_norm must have one value per bucket")
    if total_norm is not None and (total_norm.dtype != torch.float64 or total_norm.numel() < nb):
        raise ValueError("total_norm must be a float64 tensor of one entry per bucket")
    if n == 0:
        return total_norm
    arr = _grad_descs(grads, buckets)
    mx = (ctypes.c_double * nb)(*[float(v) for v in max_norm])
    _check(_lib.dmuon_clip_grad_norm_noalloc(arr, n, nb, mx, float(norm_type),
                                             total_norm.data_ptr() if total_norm is not None else None,
                                             _stream(stream, grads[0].device)), "dmuon_clip_grad_norm_noalloc")
    return total_norm


def dmuon_clip_coefficients(grads: List[torch.Tensor], max_norm, *, norm_type: float = 2.0,
                            buckets: Optional[Sequence[int]] = None, total_norm: Optional[torch.Tensor] = None,
                            coefs: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """Per-bucket clipping coefficients (float64, on the device) without
    scaling the gradients; for dmuon_step(..., grad_scale=...)."""
    n = len(grads)
    if buckets is None:
        buckets = [0] * n
    nb = (max(buckets) + 1) if n else 1
    if isinstance(max_norm, (int, float)):
        max_norm = [float(max_norm)] * nb
    nb = max(nb, len(max_norm))
    if len(max_norm) != nb or len(buckets) != n:
        raise ValueError("one max_norm per bucket and one bucket per gradient")
    arr = (dmuon_grad_t * max(n, 1))()
    for i, g in enumerate(grads):
        if not g.is_contiguous():
            raise ValueError(f"grads[{i}] must be contiguous")
        arr[i].numel, arr[i].grad, arr[i].dtype, arr[i].bucket = g.numel(), g.data_ptr(), _dtype(g), int(buckets[i])
    device = grads[0].device if n else torch.device("cpu")
    if n == 0:
        return coefs if coefs is not None else torch.ones(nb, dtype=torch.float64, device=device)
    if coefs is None:
        with torch.cuda.stream(_torch_stream(stream, device)):
            coefs = torch.ones(nb, dtype=torch.float64, device=device)
    mx = (ctypes.c_double * nb)(*[float(v) for v in max_norm])
    nbytes = int(_lib.dmuon_clip_workspace_size(arr, n, nb))
    ws, wsb = _workspace(nbytes, device, workspace, stream)
    _check(_lib.dmuon_clip_coefficients(arr, n, nb, mx, float(norm_type),
                                        total_norm.data_ptr() if total_norm is not None else None,
                                        coefs.data_ptr(), ws.data_ptr() if ws is not None else None, wsb,
                                        _stream(stream, device)), "dmuon_clip_coefficients")
    return coefs


def dmuon_plan_describe(shapes: Sequence[Sequence[int]], **hp) -> dict:
    """The launch plan of these shapes (host only, no device needed)."""
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[int(s[0]) for s in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[int(s[1]) for s in shapes])
    h, _keep = _hparams(**hp)
    need = _lib.dmuon_plan_describe(rows, cols, n, ctypes.byref(h), None, 0)
    if need < 0:
        raise DmuonError(int(need), "dmuon_plan_describe")
    buf = ctypes.create_string_buffer(int(need) + 1)
    _lib.dmuon_plan_describe(rows, cols, n, ctypes.byref(h), buf, int(need) + 1)
    return json.loads(buf.value.decode())


def dmuon_profile_begin() -> None:
    """Start bracketing every library launch with HIP events."""
    _check(_lib.dmuon_profile_begin(), "dmuon_profile_begin")


def dmuon_profile_end() -> dict:
    """Stop profiling; per kernel kind: launches, summed ms, algorithmic flops and bytes."""
    need = _lib.dmuon_profile_end(None, 0)      # closes the window, keeps the report
    if need < 0:
        raise DmuonError(int(need), "dmuon_profile_end")
    buf = ctypes.create_string_buffer(int(need) + 1)
    _lib.dmuon_profile_end(buf, int(need) + 1)  # copies the kept report
    return json.loads(buf.value.decode())
