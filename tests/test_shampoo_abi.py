"""The Shampoo entry points on the CPU: every argument check returns its status
before anything is enqueued (none of these calls reaches the HIP runtime), and
the workspace size follows the documented buffer plan."""
import ctypes
import math

import pytest

import matrix_optimizers_amd as mo
from matrix_optimizers_amd import _binding as B

OK, INVALID, UNSUPPORTED, WS_SMALL, ALIAS = 0, -1, -2, -3, -4
GiB = 1 << 30
BASE = 1 << 44


def desc(rows=64, cols=96, k=0, **kw):
    d = dict(W=BASE + (5 * k) * GiB, G=BASE + (5 * k + 1) * GiB, L=BASE + (5 * k + 2) * GiB,
             R=BASE + (5 * k + 3) * GiB)
    d.update(kw)
    return mo.shampoo_descriptor(rows, cols, **d)


def step(descs, hp=None, ws=BASE + 200 * GiB, ws_bytes=1 << 40, n=None, hp_ptr=True):
    lib = mo.load_library()
    arr, cnt = B._sh_array(descs)
    hp = hp or mo.shampoo_hparams()
    return lib.shampoo_owner_step(arr, cnt if n is None else n, ctypes.byref(hp) if hp_ptr else None,
                                  ctypes.c_void_p(ws), ws_bytes, None)


def test_noop_cases_return_ok_without_hip():
    lib = mo.load_library()
    assert lib.shampoo_owner_step(None, 0, ctypes.byref(mo.shampoo_hparams()), None, 0, None) == OK
    assert step([desc(0, 10), desc(10, 0, k=1), desc(0, 0, k=2)], ws=0, ws_bytes=0) == OK


@pytest.mark.parametrize("kw", [dict(root_iters=0), dict(root_iters=101), dict(root_iters=-3),
                                dict(lr=math.nan), dict(weight_decay=math.inf)])
def test_bad_hyperparameters(kw):
    assert step([desc()], hp=mo.shampoo_hparams(**kw)) == INVALID


def test_null_arguments():
    lib = mo.load_library()
    assert lib.shampoo_owner_step(None, 1, ctypes.byref(mo.shampoo_hparams()), None, 0, None) == INVALID
    assert step([desc()], hp_ptr=False) == INVALID
    assert step([desc()], n=-1) == INVALID
    for k in ("W", "G", "L", "R"):
        assert step([desc(**{k: 0})]) == INVALID, k


@pytest.mark.parametrize("d,code", [
    (dict(rows=-1), INVALID), (dict(cols=-3), INVALID),
    (dict(ld_w=50), INVALID), (dict(ld_g=95), INVALID), (dict(ld_l=63), INVALID),
    (dict(ld_r=95), INVALID), (dict(ld_u=1, update_out=BASE + 150 * GiB), INVALID),
    (dict(ld_r=-1), INVALID), (dict(w_dtype=3), UNSUPPORTED), (dict(g_dtype=9), UNSUPPORTED),
    (dict(rows=(1 << 23) + 1, cols=1), UNSUPPORTED),
    (dict(rows=1, cols=(1 << 16) + 1), UNSUPPORTED),        # a root side beyond 2^16
])
def test_bad_descriptors(d, code):
    args = dict(rows=64, cols=96)
    args.update(d)
    rows, cols = args.pop("rows"), args.pop("cols")
    assert step([desc(rows, cols, **args)]) == code


def test_aliasing():
    # L overlapping W, R overlapping another matrix's G, update_out over the workspace
    assert step([desc(L=BASE + 10)]) == ALIAS
    assert step([desc(), desc(k=1, R=BASE + 1 * GiB + 64)]) == ALIAS
    assert step([desc(update_out=BASE + 200 * GiB + 4096)]) == ALIAS
    # L is rows x rows with the default stride rows: 64 x 64 floats from its start
    assert step([desc(L=BASE + 64 * 96 * 4 - 4)]) == ALIAS


def test_workspace_size_and_check():
    hp = mo.shampoo_hparams()
    d = [desc(300, 200), desc(1, 700, k=1)]
    need = mo.shampoo_workspace_bytes(d, hp)
    pad = lambda x: (x + 255) // 256 * 256
    bufs = 0
    for r, c in ((300, 200), (1, 700)):
        bufs += 3 * pad(r) * pad(c) * 4 + 7 * 4 * (pad(r) ** 2 + pad(c) ** 2)
    assert bufs < need < bufs + (1 << 20)   # plus work list, partials, scales and slack
    assert step(d, ws_bytes=need - 1) == WS_SMALL
    assert step(d, ws=0, ws_bytes=need) == WS_SMALL


def test_planning_limits_fail_fast():
    """A 1 x 2^16 matrix (a 2^16-sided right root) still plans quickly; a
    bucket whose roots exceed 2^26 tiles is refused before planning."""
    import time
    t0 = time.perf_counter()
    need = mo.shampoo_workspace_bytes([desc(1, 1 << 16)], mo.shampoo_hparams())
    assert need > 7 * 4 * (1 << 32)
    many = [desc(1 << 16, 1 << 16, k=k) for k in range(400)]   # 400 x 3 x 2^16 tiles > 2^26
    with pytest.raises(mo.MoError):
        mo.shampoo_workspace_bytes(many, mo.shampoo_hparams())
    assert time.perf_counter() - t0 < 30
