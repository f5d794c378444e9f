"""The SOAP entry points on the CPU: every argument check returns its status
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
    d = dict(W=BASE + (7 * k) * GiB, G=BASE + (7 * k + 1) * GiB, L=BASE + (7 * k + 2) * GiB,
             R=BASE + (7 * k + 3) * GiB, M=BASE + (7 * k + 4) * GiB, V=BASE + (7 * k + 5) * GiB)
    ld = {key: kw.pop(key) for key in list(kw) if key.startswith("ld_")}
    d.update(kw)
    return mo.soap_descriptor(rows, cols, **d, **ld)


def step(descs, hp=None, ws=BASE + 300 * GiB, ws_bytes=1 << 40, n=None, hp_ptr=True):
    lib = mo.load_library()
    arr, cnt = B._so_array(descs)
    hp = hp or mo.soap_hparams()
    return lib.soap_owner_step(arr, cnt if n is None else n, ctypes.byref(hp) if hp_ptr else None,
                               ctypes.c_void_p(ws), ws_bytes, None)


def test_noop_cases_return_ok_without_hip():
    lib = mo.load_library()
    assert lib.soap_owner_step(None, 0, ctypes.byref(mo.soap_hparams()), None, 0, None) == OK
    assert step([desc(0, 10), desc(10, 0, k=1), desc(0, 0, k=2)], ws=0, ws_bytes=0) == OK


@pytest.mark.parametrize("kw", [dict(sweeps=0), dict(sweeps=101), dict(step=0), dict(step=-2),
                                dict(warm_start=2), dict(warm_start=-1),
                                dict(lr=math.nan), dict(weight_decay=math.inf), dict(beta1=1.0),
                                dict(beta2=-0.1), dict(eps=-1e-8), dict(eps=math.nan)])
def test_bad_hyperparameters(kw):
    assert step([desc()], hp=mo.soap_hparams(**kw)) == INVALID


def test_null_arguments():
    lib = mo.load_library()
    assert lib.soap_owner_step(None, 1, ctypes.byref(mo.soap_hparams()), None, 0, None) == INVALID
    assert step([desc()], hp_ptr=False) == INVALID
    assert step([desc()], n=-1) == INVALID
    for k in ("W", "G", "L", "R", "M", "V"):
        assert step([desc(**{k: 0})]) == INVALID, k


@pytest.mark.parametrize("d,code", [
    (dict(rows=-1), INVALID), (dict(cols=-3), INVALID),
    (dict(ld_w=50), INVALID), (dict(ld_g=95), INVALID), (dict(ld_l=63), INVALID),
    (dict(ld_r=95), INVALID), (dict(ld_m=95), INVALID), (dict(ld_v=10), INVALID),
    (dict(ld_u=1, update_out=BASE + 250 * GiB), INVALID), (dict(ld_m=-1), INVALID),
    (dict(w_dtype=3), UNSUPPORTED), (dict(g_dtype=9), UNSUPPORTED),
    (dict(rows=16385, cols=1), UNSUPPORTED), (dict(rows=1, cols=16385), UNSUPPORTED),
])
def test_bad_descriptors(d, code):
    rows, cols = d.pop("rows", 64), d.pop("cols", 96)
    assert step([desc(rows, cols, **d)]) == code


def test_workspace_checks_and_size():
    d = [desc(100, 70)]
    hp = mo.soap_hparams()
    need = mo.soap_workspace_bytes(d, hp)
    # per matrix four fp32 r_pad x c_pad buffers; per side one fp64 and two fp32
    # m_pad^2 buffers (A; the accumulated and the sorted eigenvectors), m_pad / 64
    # fp64 pair rotations of 64 x 64, the permutation, the final-sweep rotation
    # flags (one word per pair slot) and the word that marks E32 as written
    # (each region 256-aligned)
    mats = 4 * 128 * 128 * 4
    side = lambda m: (m * m * 8 + 2 * m * m * 4 + (m // 64) * 64 * 64 * 8 + max(m * 4, 256)
                      + max((m // 64) * 4, 256) + 256)
    assert need >= mats + 2 * side(128)
    assert need <= mats + 2 * side(128) + 4096
    assert step(d, ws_bytes=need - 1) == WS_SMALL
    assert step(d, ws=0) == WS_SMALL
    assert mo.soap_workspace_bytes([desc(8192, 8192)], hp) > 3 * 8192 * 8192 * 8


def test_aliasing_is_rejected():
    a = desc()
    assert step([a, desc(k=1, W=a.G)]) == ALIAS          # a written W over another's G
    assert step([desc(V=BASE + 2 * GiB + 8)]) == ALIAS  # V inside L
    assert step([desc()], ws=BASE + 4 * GiB) == ALIAS    # workspace over M


def test_rotation_item_limit_fails_fast():
    """A bucket whose rotation tiles would overflow the 32-bit item counts is
    refused on the host (2^30 tiles of 64 x 64; an 8192-sided matrix has
    2 x (128 x 129 / 2 + 128^2) = 49280)."""
    many = [desc(8192, 8192, k=k) for k in range(21790)]
    assert mo.soap_workspace_bytes(many[:100], mo.soap_hparams()) > 0
    with pytest.raises(mo.MoError):
        mo.soap_workspace_bytes(many, mo.soap_hparams())


def converged(descs, hp=None, ws=BASE + 300 * GiB, ws_bytes=1 << 40, out=True):
    lib = mo.load_library()
    arr, cnt = B._so_array(descs)
    hp = hp or mo.soap_hparams()
    buf = (ctypes.c_int32 * max(2 * cnt, 1))(*([-7] * max(2 * cnt, 1)))
    st = lib.soap_converged(arr, cnt, ctypes.byref(hp), ctypes.c_void_p(ws), ws_bytes,
                            buf if out else None, None)
    return st, list(buf)


def test_converged_argument_checks_without_hip():
    """The convergence query checks its arguments before touching the device:
    bad hyperparameters, a missing output array, a small workspace; a bucket
    of empty descriptors reports zeros."""
    assert converged([desc()], hp=mo.soap_hparams(sweeps=0))[0] == INVALID
    assert converged([desc()], out=False)[0] == INVALID
    assert converged([desc()], ws_bytes=1024)[0] == WS_SMALL
    assert converged([desc()], ws=0)[0] == WS_SMALL
    st, buf = converged([desc(0, 10), desc(10, 0, k=1)], ws=0, ws_bytes=0)
    assert st == OK and buf == [0, 0, 0, 0]
