"""ctypes binding of ``libmo.so`` (the C ABI declared in ``include/mo.h``).

Argument marshalling only: every step of the optimizer runs in the library's
HIP kernels.  PyTorch is used for device memory (the workspace) and for the
current HIP stream.  If the library is missing this module raises; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmo.so")

MO_OK = 0
MO_ERR_INVALID_ARG = -1
MO_ERR_UNSUPPORTED = -2
MO_ERR_WORKSPACE_TOO_SMALL = -3
MO_ERR_ALIAS = -4
MO_ERR_HIP = -5

MO_F32 = 0
MO_BF16 = 1
DTYPES = {"f32": MO_F32, "float32": MO_F32, "bf16": MO_BF16, "bfloat16": MO_BF16}

LR_ADJUST = {"original": 0, "match_rms_adamw": 1, "none": 2}

PHASES = ["momentum", "norm", "gram", "poly", "update", "apply", "adamw", "copy", "update_last",
          "sh_layout", "sh_stats", "sh_rootprep", "sh_root", "sh_left", "sh_right",
          "so_prep", "so_stats", "so_solve", "so_apply", "so_sort", "so_products", "so_warm"]


class MoError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class MoMatrix(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("G", ctypes.c_void_p), ("M", ctypes.c_void_p),
                ("update_out", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld_w", ctypes.c_int64), ("ld_g", ctypes.c_int64), ("ld_m", ctypes.c_int64),
                ("ld_u", ctypes.c_int64),
                ("w_dtype", ctypes.c_int32), ("g_dtype", ctypes.c_int32)]


class MoMuonHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("momentum", ctypes.c_float), ("nesterov", ctypes.c_int32),
                ("ns_steps", ctypes.c_int32), ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float),
                ("ns_c", ctypes.c_float), ("eps", ctypes.c_float), ("lr_adjust", ctypes.c_int32),
                ("ns_dtype", ctypes.c_int32)]


class MoShampooMatrix(ctypes.Structure):
    """mo_shampoo_matrix of include/mo.h."""
    _fields_ = [("W", ctypes.c_void_p), ("G", ctypes.c_void_p), ("L", ctypes.c_void_p),
                ("R", ctypes.c_void_p), ("update_out", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld_w", ctypes.c_int64), ("ld_g", ctypes.c_int64), ("ld_l", ctypes.c_int64),
                ("ld_r", ctypes.c_int64), ("ld_u", ctypes.c_int64),
                ("w_dtype", ctypes.c_int32), ("g_dtype", ctypes.c_int32)]


class MoShampooHParams(ctypes.Structure):
    """mo_shampoo_hparams of include/mo.h."""
    _fields_ = [("lr", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("root_iters", ctypes.c_int32)]


class MoSoapMatrix(ctypes.Structure):
    """mo_soap_matrix of include/mo.h."""
    _fields_ = [("W", ctypes.c_void_p), ("G", ctypes.c_void_p), ("L", ctypes.c_void_p),
                ("R", ctypes.c_void_p), ("M", ctypes.c_void_p), ("V", ctypes.c_void_p),
                ("update_out", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld_w", ctypes.c_int64), ("ld_g", ctypes.c_int64), ("ld_l", ctypes.c_int64),
                ("ld_r", ctypes.c_int64), ("ld_m", ctypes.c_int64), ("ld_v", ctypes.c_int64),
                ("ld_u", ctypes.c_int64), ("w_dtype", ctypes.c_int32), ("g_dtype", ctypes.c_int32)]


class MoSoapHParams(ctypes.Structure):
    """mo_soap_hparams of include/mo.h."""
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int32),
                ("sweeps", ctypes.c_int32), ("warm_start", ctypes.c_int32)]


_lib = None

EXPORTS = ["muon_workspace_bytes", "muon_build_worklist", "muon_owner_step", "adamw_tail_step",
           "mo_status_string", "mo_profile_enable", "mo_profile_read", "mo_device_copy",
           "mo_plan_owners", "mo_plan_score", "mo_plan_layout", "shampoo_workspace_bytes",
           "shampoo_owner_step", "soap_workspace_bytes", "soap_owner_step", "soap_converged",
           "muon_owner_step_noalloc"]

ROLE_MATRIX, ROLE_TAIL = 0, 1
PLAN_POLICIES = {"role_greedy": 0, "scope_greedy": 1, "cost_aware": 2}


class MoRole(ctypes.Structure):
    """mo_role of include/mo.h."""
    _fields_ = [("block", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmo.so once; raise loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m matrix_optimizers_amd.build`"
                           " (there is no non-HIP fallback)")
    # The binding hands torch's device memory and streams to the library, so
    # both must run on one HIP runtime.  torch ships its own, under the same
    # soname as the system's that libmo.so is linked against: whichever loads
    # first serves the process.  Loaded before torch, libmo.so would put torch
    # on the system runtime, where the step's launches fail; torch goes first.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.muon_workspace_bytes.argtypes = [P(MoMatrix), ctypes.c_int32, P(MoMuonHParams),
                                         P(ctypes.c_size_t)]
    lib.muon_build_worklist.argtypes = [P(MoMatrix), ctypes.c_int32, P(MoMuonHParams),
                                        ctypes.c_void_p, P(ctypes.c_size_t)]
    lib.muon_owner_step.argtypes = [P(MoMatrix), ctypes.c_int32, P(MoMuonHParams),
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.muon_owner_step_noalloc.argtypes = [P(MoMatrix), ctypes.c_int32, P(MoMuonHParams), ctypes.c_void_p]
    lib.adamw_tail_step.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int64] + \
        [ctypes.c_float] * 5 + [ctypes.c_void_p]
    lib.mo_status_string.argtypes = [ctypes.c_int32]
    lib.mo_status_string.restype = ctypes.c_char_p
    lib.mo_profile_enable.argtypes = [ctypes.c_int32]
    lib.mo_profile_read.argtypes = [P(ctypes.c_double), P(ctypes.c_int64)]
    lib.mo_device_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p]
    lib.mo_plan_owners.argtypes = [P(MoRole), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int64, P(ctypes.c_int32)]
    lib.mo_plan_score.argtypes = [P(MoRole), ctypes.c_int32, ctypes.c_int32, P(ctypes.c_int32),
                                  P(ctypes.c_double), P(ctypes.c_double), ctypes.c_int32,
                                  P(ctypes.c_double), P(ctypes.c_double)]
    lib.mo_plan_layout.argtypes = [P(MoRole), ctypes.c_int32, ctypes.c_int32, P(ctypes.c_int32),
                                   P(ctypes.c_int64)]
    lib.shampoo_workspace_bytes.argtypes = [P(MoShampooMatrix), ctypes.c_int32, P(MoShampooHParams),
                                            P(ctypes.c_size_t)]
    lib.shampoo_owner_step.argtypes = [P(MoShampooMatrix), ctypes.c_int32, P(MoShampooHParams),
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.soap_workspace_bytes.argtypes = [P(MoSoapMatrix), ctypes.c_int32, P(MoSoapHParams),
                                         P(ctypes.c_size_t)]
    lib.soap_owner_step.argtypes = [P(MoSoapMatrix), ctypes.c_int32, P(MoSoapHParams),
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.soap_converged.argtypes = [P(MoSoapMatrix), ctypes.c_int32, P(MoSoapHParams), ctypes.c_void_p,
                                   ctypes.c_size_t, P(ctypes.c_int32), ctypes.c_void_p]
    for name in ("muon_workspace_bytes", "muon_build_worklist", "muon_owner_step",
                 "adamw_tail_step", "mo_profile_enable", "mo_profile_read", "mo_device_copy",
                 "mo_plan_owners", "mo_plan_score", "mo_plan_layout", "shampoo_workspace_bytes",
                 "shampoo_owner_step", "soap_workspace_bytes", "soap_owner_step", "soap_converged",
                 "muon_owner_step_noalloc"):
        getattr(lib, name).restype = ctypes.c_int32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mo_status_string(int(status)).decode()


mo_status_string = status_string


def _check(status: int, where: str) -> None:
    if status != MO_OK:
        raise MoError(status, where)


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

def hparams(lr: float = 0.02, weight_decay: float = 0.01, momentum: float = 0.95,
            nesterov: bool = True, ns_steps: int = 5,
            ns_coefficients: Tuple[float, float, float] = (3.4445, -4.7750, 2.0315),
            eps: float = 1e-7, adjust_lr_fn: str = "original",
            ns_dtype: str = "bf16") -> MoMuonHParams:
    a, b, c = ns_coefficients
    return MoMuonHParams(lr=lr, weight_decay=weight_decay, momentum=momentum,
                         nesterov=1 if nesterov else 0, ns_steps=int(ns_steps), ns_a=a, ns_b=b,
                         ns_c=c, eps=eps, lr_adjust=LR_ADJUST[adjust_lr_fn],
                         ns_dtype=DTYPES[ns_dtype])


def descriptor(rows: int, cols: int, W: int = 0, G: int = 0, M: int = 0, update_out: int = 0,
               w_dtype: str = "bf16", g_dtype: str = "bf16", ld_w: int = 0, ld_g: int = 0,
               ld_m: int = 0, ld_u: int = 0) -> MoMatrix:
    """A raw descriptor from integer addresses (host-side planning and tests)."""
    return MoMatrix(W=W or None, G=G or None, M=M or None, update_out=update_out or None,
                    rows=rows, cols=cols, ld_w=ld_w, ld_g=ld_g, ld_m=ld_m, ld_u=ld_u,
                    w_dtype=DTYPES[w_dtype] if isinstance(w_dtype, str) else int(w_dtype),
                    g_dtype=DTYPES[g_dtype] if isinstance(g_dtype, str) else int(g_dtype))


def _array(descs: Sequence[MoMatrix]):
    n = len(descs)
    arr = (MoMatrix * max(n, 1))()
    for i, d in enumerate(descs):
        arr[i] = d
    return arr, n


def workspace_bytes(descs: Sequence[MoMatrix], hp: MoMuonHParams) -> int:
    lib = load_library()
    arr, n = _array(descs)
    out = ctypes.c_size_t(0)
    _check(lib.muon_workspace_bytes(arr, n, ctypes.byref(hp), ctypes.byref(out)),
           "muon_workspace_bytes")
    return int(out.value)


def build_worklist(descs: Sequence[MoMatrix], hp: MoMuonHParams) -> bytes:
    lib = load_library()
    arr, n = _array(descs)
    size = ctypes.c_size_t(0)
    _check(lib.muon_build_worklist(arr, n, ctypes.byref(hp), None, ctypes.byref(size)),
           "muon_build_worklist")
    buf = ctypes.create_string_buffer(size.value)
    _check(lib.muon_build_worklist(arr, n, ctypes.byref(hp), buf, ctypes.byref(size)),
           "muon_build_worklist")
    return buf.raw[: size.value]


muon_workspace_bytes = workspace_bytes
muon_build_worklist = build_worklist


# ---------------------------------------------------------------------------
# torch-facing entry points
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MO_F32
    if t.dtype == torch.bfloat16:
        return MO_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _row_stride(t) -> int:
    if t.dim() != 2:
        raise ValueError("matrices must be 2D")
    if t.numel() and t.stride(1) != 1:
        raise ValueError("matrices must be row-major with unit column stride")
    return int(t.stride(0)) if t.numel() else 0


def tensor_descriptor(W, G, M, update_out=None) -> MoMatrix:
    torch = _torch()
    if W.shape != G.shape or W.shape != M.shape:
        raise ValueError("W, G, M shapes differ")
    if M.dtype != torch.float32:
        raise TypeError("momentum buffers are float32")
    dev = W.device
    for t in (G, M) + ((update_out,) if update_out is not None else ()):
        if t.device != dev:
            raise ValueError("W, G, M, update_out must be on one device")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    rows, cols = W.shape
    if update_out is not None:
        if update_out.shape != W.shape or update_out.dtype != torch.float32:
            raise ValueError("update_out must be float32 and shaped like W")
    return MoMatrix(W=W.data_ptr() or None, G=G.data_ptr() or None, M=M.data_ptr() or None,
                    update_out=(update_out.data_ptr() if update_out is not None else None),
                    rows=rows, cols=cols, ld_w=_row_stride(W), ld_g=_row_stride(G),
                    ld_m=_row_stride(M), ld_u=_row_stride(update_out) if update_out is not None else 0,
                    w_dtype=_dtype_code(W), g_dtype=_dtype_code(G))


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _workspace_for(nbytes: int, mats, stream):
    """A uint8 workspace tensor allocated on the stream the step launches on.

    The caching allocator ties a block to the stream current at allocation and
    hands it out again, once freed, in that stream's order; a workspace made on
    another stream than the launch stream could be reused by later work there
    while the step's kernels still read it."""
    torch = _torch()
    dev = mats[0][0].device if mats else torch.device("cuda")
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(_stream_handle(stream), device=dev)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def _record_launch_stream(workspace, alloc_stream: int, stream) -> None:
    """A reusable step's workspace was allocated on ``alloc_stream``; when a
    call launches on another stream, that stream is recorded on the block, so
    the caching allocator does not hand it out again (after the step object is
    dropped) before the work queued there has finished."""
    torch = _torch()
    handle = _stream_handle(stream)
    if handle == alloc_stream:
        return
    if isinstance(stream, torch.cuda.Stream):
        workspace.record_stream(stream)
    else:
        workspace.record_stream(torch.cuda.ExternalStream(handle, device=workspace.device))


def muon_owner_step(mats: Sequence[Tuple], *, update_out: Optional[Sequence] = None,
                    workspace=None, stream=None, **hp_kwargs) -> None:
    """One Muon step over a bucket of (W, G, M) tensors, in place.

    hp_kwargs: lr, weight_decay, momentum, nesterov, ns_steps, ns_coefficients,
    eps, adjust_lr_fn ("original" | "match_rms_adamw" | "none"), ns_dtype
    ("bf16" | "f32").  workspace: an optional uint8 device tensor of at least
    workspace_bytes(); one is allocated on the launch stream when omitted.  A
    caller's workspace must not be freed or reused by other work until the
    step has finished on ``stream``.
    """
    lib = load_library()
    hp = hparams(**hp_kwargs)
    ups = list(update_out) if update_out is not None else [None] * len(mats)
    descs = [tensor_descriptor(W, G, M, u) for (W, G, M), u in zip(mats, ups)]
    arr, n = _array(descs)
    need = ctypes.c_size_t(0)
    _check(lib.muon_workspace_bytes(arr, n, ctypes.byref(hp), ctypes.byref(need)),
           "muon_workspace_bytes")
    if workspace is None:
        workspace = _workspace_for(int(need.value), mats, stream)
    _check(lib.muon_owner_step(arr, n, ctypes.byref(hp), ctypes.c_void_p(workspace.data_ptr()),
                               workspace.numel(), ctypes.c_void_p(_stream_handle(stream))),
           "muon_owner_step")


NOALLOC_SCRATCH_BYTES = 512 << 20   # MO_NOALLOC_SCRATCH_BYTES of include/mo.h


def muon_owner_step_noalloc(mats: Sequence[Tuple], *, update_out: Optional[Sequence] = None,
                            stream=None, **hp_kwargs) -> None:
    """muon_owner_step on the library's static per-device scratch array: no
    workspace argument and no device allocation (for callers that cannot
    allocate).  Buckets whose workspace exceeds NOALLOC_SCRATCH_BYTES are
    refused; calls that overlap in time on one device race."""
    lib = load_library()
    hp = hparams(**hp_kwargs)
    ups = list(update_out) if update_out is not None else [None] * len(mats)
    descs = [tensor_descriptor(W, G, M, u) for (W, G, M), u in zip(mats, ups)]
    arr, n = _array(descs)
    _check(lib.muon_owner_step_noalloc(arr, n, ctypes.byref(hp), ctypes.c_void_p(_stream_handle(stream))),
           "muon_owner_step_noalloc")


class MuonOwnerStep:
    """Reusable step over a fixed bucket: descriptors and workspace are prepared
    once; ``__call__`` launches the step on the current (or given) stream.
    Every call uses the one workspace: calls on different streams must not
    overlap in time."""

    def __init__(self, mats: Sequence[Tuple], update_out: Optional[Sequence] = None,
                 **hp_kwargs):
        torch = _torch()
        self.lib = load_library()
        self.hp = hparams(**hp_kwargs)
        ups = list(update_out) if update_out is not None else [None] * len(mats)
        self.descs = [tensor_descriptor(W, G, M, u) for (W, G, M), u in zip(mats, ups)]
        self.arr, self.n = _array(self.descs)
        self.bytes = workspace_bytes(self.descs, self.hp)
        dev = mats[0][0].device if mats else torch.device("cuda")
        self.workspace = torch.empty(self.bytes, dtype=torch.uint8, device=dev)
        self._alloc_stream = int(torch.cuda.current_stream(dev).cuda_stream)
        self._keep = (mats, update_out)

    def __call__(self, stream=None) -> None:
        _record_launch_stream(self.workspace, self._alloc_stream, stream)
        _check(self.lib.muon_owner_step(self.arr, self.n, ctypes.byref(self.hp),
                                        ctypes.c_void_p(self.workspace.data_ptr()),
                                        self.workspace.numel(),
                                        ctypes.c_void_p(_stream_handle(stream))),
               "muon_owner_step")


# ---------------------------------------------------------------------------
# Shampoo
# ---------------------------------------------------------------------------

def shampoo_hparams(lr: float = 1e-3, weight_decay: float = 0.0, root_iters: int = 20) -> MoShampooHParams:
    return MoShampooHParams(lr=lr, weight_decay=weight_decay, root_iters=int(root_iters))


def shampoo_descriptor(rows: int, cols: int, W: int = 0, G: int = 0, L: int = 0, R: int = 0,
                       update_out: int = 0, w_dtype="f32", g_dtype="f32", ld_w: int = 0,
                       ld_g: int = 0, ld_l: int = 0, ld_r: int = 0, ld_u: int = 0) -> MoShampooMatrix:
    """A raw descriptor from integer addresses (host-side planning and tests)."""
    code = lambda d: DTYPES[d] if isinstance(d, str) else int(d)
    return MoShampooMatrix(W=W or None, G=G or None, L=L or None, R=R or None,
                           update_out=update_out or None, rows=rows, cols=cols, ld_w=ld_w, ld_g=ld_g,
                           ld_l=ld_l, ld_r=ld_r, ld_u=ld_u, w_dtype=code(w_dtype), g_dtype=code(g_dtype))


def shampoo_tensor_descriptor(W, G, L, R, update_out=None) -> MoShampooMatrix:
    torch = _torch()
    if W.shape != G.shape:
        raise ValueError("W and G shapes differ")
    rows, cols = W.shape
    if tuple(L.shape) != (rows, rows) or tuple(R.shape) != (cols, cols):
        raise ValueError("L must be rows x rows and R cols x cols")
    if L.dtype != torch.float32 or R.dtype != torch.float32:
        raise TypeError("statistics are float32")
    dev = W.device
    for t in (G, L, R) + ((update_out,) if update_out is not None else ()):
        if t.device != dev:
            raise ValueError("W, G, L, R, update_out must be on one device")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    if update_out is not None and (update_out.shape != W.shape or update_out.dtype != torch.float32):
        raise ValueError("update_out must be float32 and shaped like W")
    return MoShampooMatrix(W=W.data_ptr() or None, G=G.data_ptr() or None, L=L.data_ptr() or None,
                           R=R.data_ptr() or None,
                           update_out=(update_out.data_ptr() if update_out is not None else None),
                           rows=rows, cols=cols, ld_w=_row_stride(W), ld_g=_row_stride(G),
                           ld_l=_row_stride(L), ld_r=_row_stride(R),
                           ld_u=_row_stride(update_out) if update_out is not None else 0,
                           w_dtype=_dtype_code(W), g_dtype=_dtype_code(G))


def _sh_array(descs: Sequence[MoShampooMatrix]):
    n = len(descs)
    arr = (MoShampooMatrix * max(n, 1))()
    for i, d in enumerate(descs):
        arr[i] = d
    return arr, n


def shampoo_workspace_bytes(descs: Sequence[MoShampooMatrix], hp: MoShampooHParams) -> int:
    lib = load_library()
    arr, n = _sh_array(descs)
    out = ctypes.c_size_t(0)
    _check(lib.shampoo_workspace_bytes(arr, n, ctypes.byref(hp), ctypes.byref(out)),
           "shampoo_workspace_bytes")
    return int(out.value)


class ShampooOwnerStep:
    """Reusable Shampoo step over a fixed bucket of (W, G, L, R) tensors:
    descriptors and workspace are prepared once; ``__call__`` launches the step
    (W, L, R updated in place) on the current (or given) stream.  Every call
    uses the one workspace: calls on different streams must not overlap in
    time."""

    def __init__(self, mats: Sequence[Tuple], update_out: Optional[Sequence] = None, **hp_kwargs):
        torch = _torch()
        self.lib = load_library()
        self.hp = shampoo_hparams(**hp_kwargs)
        ups = list(update_out) if update_out is not None else [None] * len(mats)
        self.descs = [shampoo_tensor_descriptor(W, G, L, R, u) for (W, G, L, R), u in zip(mats, ups)]
        self.arr, self.n = _sh_array(self.descs)
        self.bytes = shampoo_workspace_bytes(self.descs, self.hp)
        dev = mats[0][0].device if mats else torch.device("cuda")
        self.workspace = torch.empty(self.bytes, dtype=torch.uint8, device=dev)
        self._alloc_stream = int(torch.cuda.current_stream(dev).cuda_stream)
        self._keep = (mats, update_out)

    def __call__(self, stream=None) -> None:
        _record_launch_stream(self.workspace, self._alloc_stream, stream)
        _check(self.lib.shampoo_owner_step(self.arr, self.n, ctypes.byref(self.hp),
                                           ctypes.c_void_p(self.workspace.data_ptr()),
                                           self.workspace.numel(),
                                           ctypes.c_void_p(_stream_handle(stream))),
               "shampoo_owner_step")


def shampoo_owner_step(mats: Sequence[Tuple], *, update_out: Optional[Sequence] = None,
                       workspace=None, stream=None, **hp_kwargs) -> None:
    """One Shampoo step over a bucket of (W, G, L, R) tensors, in place.

    hp_kwargs: lr, weight_decay, root_iters.  L and R are the float32
    statistics (rows x rows, cols x cols), started by the caller at eps I.
    """
    lib = load_library()
    hp = shampoo_hparams(**hp_kwargs)
    ups = list(update_out) if update_out is not None else [None] * len(mats)
    descs = [shampoo_tensor_descriptor(W, G, L, R, u) for (W, G, L, R), u in zip(mats, ups)]
    arr, n = _sh_array(descs)
    need = shampoo_workspace_bytes(descs, hp)
    if workspace is None:
        workspace = _workspace_for(need, mats, stream)
    _check(lib.shampoo_owner_step(arr, n, ctypes.byref(hp), ctypes.c_void_p(workspace.data_ptr()),
                                  workspace.numel(), ctypes.c_void_p(_stream_handle(stream))),
           "shampoo_owner_step")


# ---------------------------------------------------------------------------
# SOAP
# ---------------------------------------------------------------------------

def soap_hparams(lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                 weight_decay: float = 0.0, step: int = 1, sweeps: int = 14,
                 warm_start: int = 0) -> MoSoapHParams:
    return MoSoapHParams(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay,
                         step=int(step), sweeps=int(sweeps), warm_start=int(warm_start))


def soap_descriptor(rows: int, cols: int, W: int = 0, G: int = 0, L: int = 0, R: int = 0, M: int = 0,
                    V: int = 0, update_out: int = 0, w_dtype="f32", g_dtype="f32", **ld) -> MoSoapMatrix:
    """A raw descriptor from integer addresses (host-side checks and tests); ld_* strides by name."""
    code = lambda d: DTYPES[d] if isinstance(d, str) else int(d)
    return MoSoapMatrix(W=W or None, G=G or None, L=L or None, R=R or None, M=M or None, V=V or None,
                        update_out=update_out or None, rows=rows, cols=cols, w_dtype=code(w_dtype),
                        g_dtype=code(g_dtype), **ld)


def soap_tensor_descriptor(W, G, L, R, M, V, update_out=None) -> MoSoapMatrix:
    torch = _torch()
    if W.shape != G.shape or M.shape != W.shape or V.shape != W.shape:
        raise ValueError("W, G, M and V must have one shape")
    rows, cols = W.shape
    if tuple(L.shape) != (rows, rows) or tuple(R.shape) != (cols, cols):
        raise ValueError("L must be rows x rows and R cols x cols")
    for t in (L, R, M, V):
        if t.dtype != torch.float32:
            raise TypeError("statistics and moments are float32")
    dev = W.device
    for t in (G, L, R, M, V) + ((update_out,) if update_out is not None else ()):
        if t.device != dev:
            raise ValueError("W, G, L, R, M, V, update_out must be on one device")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    if update_out is not None and (update_out.shape != W.shape or update_out.dtype != torch.float32):
        raise ValueError("update_out must be float32 and shaped like W")
    ptr = lambda t: t.data_ptr() or None
    return MoSoapMatrix(W=ptr(W), G=ptr(G), L=ptr(L), R=ptr(R), M=ptr(M), V=ptr(V),
                        update_out=(update_out.data_ptr() if update_out is not None else None),
                        rows=rows, cols=cols, ld_w=_row_stride(W), ld_g=_row_stride(G),
                        ld_l=_row_stride(L), ld_r=_row_stride(R), ld_m=_row_stride(M),
                        ld_v=_row_stride(V),
                        ld_u=_row_stride(update_out) if update_out is not None else 0,
                        w_dtype=_dtype_code(W), g_dtype=_dtype_code(G))


def _so_array(descs: Sequence[MoSoapMatrix]):
    n = len(descs)
    arr = (MoSoapMatrix * max(n, 1))()
    for i, d in enumerate(descs):
        arr[i] = d
    return arr, n


def soap_workspace_bytes(descs: Sequence[MoSoapMatrix], hp: MoSoapHParams) -> int:
    lib = load_library()
    arr, n = _so_array(descs)
    out = ctypes.c_size_t(0)
    _check(lib.soap_workspace_bytes(arr, n, ctypes.byref(hp), ctypes.byref(out)), "soap_workspace_bytes")
    return int(out.value)


class SoapOwnerStep:
    """Reusable SOAP step over a fixed bucket of (W, G, L, R, M, V) tensors:
    descriptors and workspace are prepared once; ``__call__(step)`` launches
    one step (W, L, R, M, V updated in place) on the current (or given)
    stream.  Every call uses the one workspace: calls on different streams
    must not overlap in time.  With ``warm_start=True`` every call after the
    first starts the eigensolver from the eigenbases the previous call left
    in the workspace (the same eigendecomposition, by fewer rotating sweeps)."""

    def __init__(self, mats: Sequence[Tuple], update_out: Optional[Sequence] = None,
                 warm_start: bool = False, **hp_kwargs):
        torch = _torch()
        self.lib = load_library()
        self.hp_kwargs = dict(hp_kwargs)
        self.hp = soap_hparams(**hp_kwargs)
        self.warm_start = bool(warm_start)
        self._has_bases = False
        ups = list(update_out) if update_out is not None else [None] * len(mats)
        self.descs = [soap_tensor_descriptor(*mat, u) for mat, u in zip(mats, ups)]
        self.arr, self.n = _so_array(self.descs)
        self.bytes = soap_workspace_bytes(self.descs, self.hp)
        dev = mats[0][0].device if mats else torch.device("cuda")
        self.workspace = torch.empty(self.bytes, dtype=torch.uint8, device=dev)
        self._alloc_stream = int(torch.cuda.current_stream(dev).cuda_stream)
        self._keep = (mats, update_out)

    def __call__(self, step: Optional[int] = None, stream=None) -> None:
        if step is not None:
            self.hp.step = int(step)
        _record_launch_stream(self.workspace, self._alloc_stream, stream)
        self.hp.warm_start = int(self.warm_start and self._has_bases)
        self._has_bases = False   # until this call has returned without error
        _check(self.lib.soap_owner_step(self.arr, self.n, ctypes.byref(self.hp),
                                        ctypes.c_void_p(self.workspace.data_ptr()),
                                        self.workspace.numel(),
                                        ctypes.c_void_p(_stream_handle(stream))),
               "soap_owner_step")
        self._has_bases = True

    def rotating_pairs(self, stream=None) -> List[Tuple[int, int]]:
        """(L', R') per matrix: pair slots that still rotated in the last
        call's final Jacobi sweep (0 = converged); waits for that call."""
        out = (ctypes.c_int32 * max(2 * self.n, 1))()
        _check(self.lib.soap_converged(self.arr, self.n, ctypes.byref(self.hp),
                                       ctypes.c_void_p(self.workspace.data_ptr()), self.workspace.numel(),
                                       out, ctypes.c_void_p(_stream_handle(stream))),
               "soap_converged")
        return [(int(out[2 * i]), int(out[2 * i + 1])) for i in range(self.n)]


def soap_converged(mats: Sequence[Tuple], workspace, *, stream=None, **hp_kwargs) -> List[Tuple[int, int]]:
    """After soap_owner_step(mats, workspace=workspace, **hp_kwargs): per matrix,
    (L', R') pair slots that still rotated in the final Jacobi sweep (0 =
    converged).  Waits for the step on ``stream``."""
    lib = load_library()
    hp = soap_hparams(**hp_kwargs)
    descs = [soap_tensor_descriptor(*mat) for mat in mats]
    arr, n = _so_array(descs)
    out = (ctypes.c_int32 * max(2 * n, 1))()
    _check(lib.soap_converged(arr, n, ctypes.byref(hp), ctypes.c_void_p(workspace.data_ptr()),
                              workspace.numel(), out, ctypes.c_void_p(_stream_handle(stream))),
           "soap_converged")
    return [(int(out[2 * i]), int(out[2 * i + 1])) for i in range(n)]


def soap_owner_step(mats: Sequence[Tuple], *, update_out: Optional[Sequence] = None,
                    workspace=None, stream=None, **hp_kwargs) -> None:
    """One SOAP step over a bucket of (W, G, L, R, M, V) tensors, in place.

    hp_kwargs: lr, beta1, beta2, eps, weight_decay, step (t of the bias
    corrections), sweeps (outer Jacobi sweeps), warm_start (1: start the
    eigensolver from the bases the previous step of this bucket left in
    ``workspace``; a workspace without them runs cold).  L and R are the float32
    statistics (started by the caller at eps I), M the first moment in the
    weight's frame and V the second moment in the eigenbasis (float32, zeros
    at the start).
    """
    lib = load_library()
    hp = soap_hparams(**hp_kwargs)
    ups = list(update_out) if update_out is not None else [None] * len(mats)
    descs = [soap_tensor_descriptor(*mat, u) for mat, u in zip(mats, ups)]
    arr, n = _so_array(descs)
    need = soap_workspace_bytes(descs, hp)
    if workspace is None:
        workspace = _workspace_for(need, mats, stream)
    _check(lib.soap_owner_step(arr, n, ctypes.byref(hp), ctypes.c_void_p(workspace.data_ptr()),
                               workspace.numel(), ctypes.c_void_p(_stream_handle(stream))),
           "soap_owner_step")


def adamw_tail_step(p, g, m, v, step: int, *, lr: float = 1e-3, beta1: float = 0.9,
                    beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 1e-2,
                    stream=None) -> None:
    """One AdamW step on flat fp32 device tensors p, g, m, v, in place."""
    torch = _torch()
    for t in (p, g, m, v):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("tail tensors must be contiguous float32 device tensors")
        if t.numel() != p.numel():
            raise ValueError("tail tensors differ in length")
    lib = load_library()
    _check(lib.adamw_tail_step(ctypes.c_void_p(p.data_ptr()), ctypes.c_void_p(g.data_ptr()),
                               ctypes.c_void_p(m.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                               p.numel(), int(step), lr, beta1, beta2, eps, weight_decay,
                               ctypes.c_void_p(_stream_handle(stream))),
           "adamw_tail_step")


def device_copy(dst, src, stream=None) -> None:
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("destination too small")
    _check(lib.mo_device_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                              nbytes, ctypes.c_void_p(_stream_handle(stream))), "mo_device_copy")


def profile_enable(on: bool = True) -> None:
    _check(load_library().mo_profile_enable(1 if on else 0), "mo_profile_enable")


def profile_read() -> dict:
    """Per-phase {name: (total_ms, launches)} of the launches timed since the last read."""
    ms = (ctypes.c_double * len(PHASES))()
    cnt = (ctypes.c_int64 * len(PHASES))()
    _check(load_library().mo_profile_read(ms, cnt), "mo_profile_read")
    return {name: (ms[i], cnt[i]) for i, name in enumerate(PHASES)}


# ---- owner planner (host only) ----------------------------------------------

def _roles(roles):
    """roles: sequence of (block, kind, rows, cols); kind ROLE_MATRIX / ROLE_TAIL."""
    arr = (MoRole * max(len(roles), 1))()
    for i, (b, k, r, c) in enumerate(roles):
        arr[i] = MoRole(int(b), int(k), int(r), int(c))
    return arr, len(roles)


def plan_owners(roles, world: int, policy: str = "role_greedy", block_cap: int = 0) -> list:
    """Owner rank of each role (mo_plan_owners)."""
    if policy not in PLAN_POLICIES:
        raise ValueError(f"unknown policy {policy!r}")
    arr, n = _roles(roles)
    out = (ctypes.c_int32 * max(n, 1))()
    _check(load_library().mo_plan_owners(arr, n, int(world), PLAN_POLICIES[policy], int(block_cap), out),
           "mo_plan_owners")
    return list(out[:n])


def plan_score(roles, world: int, owner) -> dict:
    """Per-rank numel and NS flops, per-block gamma_B and C_owner (mo_plan_score)."""
    arr, n = _roles(roles)
    own = (ctypes.c_int32 * max(n, 1))(*owner)
    nb = 1 + max((int(r[0]) for r in roles), default=-1)
    rn = (ctypes.c_double * world)()
    rf = (ctypes.c_double * world)()
    bg = (ctypes.c_double * max(nb, 1))()
    bc = (ctypes.c_double * max(nb, 1))()
    _check(load_library().mo_plan_score(arr, n, int(world), own, rn, rf, nb, bg, bc), "mo_plan_score")
    return {"rank_numel": list(rn), "rank_flops": list(rf), "block_gamma": list(bg[:nb]),
            "block_owner_comm": list(bc[:nb])}


def plan_layout(roles, world: int, owner) -> list:
    """Element offset of each role in its owner's block-local buffer (mo_plan_layout)."""
    arr, n = _roles(roles)
    own = (ctypes.c_int32 * max(n, 1))(*owner)
    out = (ctypes.c_int64 * max(n, 1))()
    _check(load_library().mo_plan_layout(arr, n, int(world), own, out), "mo_plan_layout")
    return list(out[:n])
