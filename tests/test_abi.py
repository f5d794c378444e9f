"""The C-ABI library on the CPU: it loads, exports every function include/mo.h
declares, and every argument check returns its status before anything is
enqueued (so none of these calls reaches the HIP runtime)."""
import ctypes
import math
import os
import re

import pytest

import matrix_optimizers_amd as mo
from matrix_optimizers_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mo.h")

OK, INVALID, UNSUPPORTED, WS_SMALL, ALIAS, HIP = 0, -1, -2, -3, -4, -5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = mo.load_library()
    names = declared_functions()
    assert {"muon_owner_step", "adamw_tail_step", "muon_workspace_bytes", "muon_build_worklist",
            "mo_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(B.EXPORTS) == set(names)


def test_status_strings():
    for code in (OK, INVALID, UNSUPPORTED, WS_SMALL, ALIAS, HIP):
        assert mo.status_string(code).startswith("MO_")
    assert "unknown" in mo.status_string(99)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError):
        B.load_library(str(tmp_path / "nope.so"))
    monkeypatch.setattr(B, "_lib", None)
    B.load_library()


def test_library_shares_torchs_hip_runtime():
    """torch ships its own HIP runtime under the system runtime's soname, and the
    first one loaded serves the whole process.  Loading the library through the
    binding, even before anything else imports torch, leaves exactly one
    libamdhip64 mapped, torch's, so the two cannot end up on different runtimes."""
    import subprocess
    import sys
    code = ("from matrix_optimizers_amd import _binding\n"
            "_binding.load_library()\n"
            "import os, torch\n"
            "tl = os.path.realpath(os.path.join(os.path.dirname(torch.__file__), 'lib'))\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(maps), all(os.path.realpath(m).startswith(tl) for m in maps))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split()[-2:] == ["1", "True"], out.stdout


GiB = 1 << 30
BASE = 1 << 44


def desc(rows=64, cols=96, k=0, **kw):
    d = dict(W=BASE + (3 * k) * GiB, G=BASE + (3 * k + 1) * GiB, M=BASE + (3 * k + 2) * GiB)
    d.update(kw)
    return mo.descriptor(rows, cols, **d)


def step(descs, hp=None, ws=BASE + 100 * GiB, ws_bytes=1 << 40, n=None, hp_ptr=True):
    lib = mo.load_library()
    arr, cnt = B._array(descs)
    hp = hp or mo.hparams()
    return lib.muon_owner_step(arr, cnt if n is None else n, ctypes.byref(hp) if hp_ptr else None,
                               ctypes.c_void_p(ws), ws_bytes, None)


def test_noop_cases_return_ok_without_hip():
    lib = mo.load_library()
    assert lib.muon_owner_step(None, 0, ctypes.byref(mo.hparams()), None, 0, None) == OK
    # all-empty bucket: every shard is a non-owner's empty view
    assert step([desc(0, 10), desc(10, 0, k=1), desc(0, 0, k=2)], ws=0, ws_bytes=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(ns_steps=-1), INVALID), (dict(eps=0.0), INVALID), (dict(eps=-1.0), INVALID),
    (dict(lr=math.nan), INVALID), (dict(weight_decay=math.inf), INVALID),
    (dict(momentum=math.nan), INVALID), (dict(ns_coefficients=(math.nan, 1, 1)), INVALID),
])
def test_bad_hyperparameters(kw, code):
    assert step([desc()], hp=mo.hparams(**kw)) == code


def test_bad_enums():
    hp = mo.hparams()
    hp.lr_adjust = 7
    assert step([desc()], hp=hp) == INVALID
    hp = mo.hparams()
    hp.ns_dtype = 5
    assert step([desc()], hp=hp) == UNSUPPORTED


def test_null_arguments():
    lib = mo.load_library()
    assert lib.muon_owner_step(None, 1, ctypes.byref(mo.hparams()), None, 0, None) == INVALID
    assert step([desc()], hp_ptr=False) == INVALID
    assert step([desc()], n=-1) == INVALID
    assert step([desc(W=0)]) == INVALID
    assert step([desc(G=0)]) == INVALID
    assert step([desc(M=0)]) == INVALID


@pytest.mark.parametrize("d,code", [
    (dict(rows=-1), INVALID), (dict(cols=-3), INVALID),
    (dict(ld_w=50), INVALID), (dict(ld_g=95), INVALID), (dict(ld_m=10), INVALID),
    (dict(ld_u=1, update_out=BASE + 50 * GiB), INVALID), (dict(ld_w=-1), INVALID),
    (dict(w_dtype=3), UNSUPPORTED), (dict(g_dtype=9), UNSUPPORTED),
    (dict(rows=(1 << 23) + 1, cols=1), UNSUPPORTED),
    (dict(rows=1 << 23, cols=1 << 14), UNSUPPORTED),       # 2^37 elements
])
def test_bad_descriptors(d, code):
    args = dict(rows=64, cols=96)
    args.update(d)
    rows, cols = args.pop("rows"), args.pop("cols")
    assert step([desc(rows, cols, **args)]) == code


def test_workspace_checks():
    d = [desc()]
    need = mo.workspace_bytes(d, mo.hparams())
    assert step(d, ws_bytes=need - 1) == WS_SMALL
    assert step(d, ws=0, ws_bytes=need) == WS_SMALL


@pytest.mark.parametrize("case", ["w_overlaps_m", "w_overlaps_other_g", "m_overlaps_other_w",
                                  "update_overlaps_g", "workspace_overlaps_w", "same_w_twice"])
def test_aliasing_is_rejected(case):
    a = dict(W=BASE, G=BASE + GiB, M=BASE + 2 * GiB)
    b = dict(W=BASE + 3 * GiB, G=BASE + 4 * GiB, M=BASE + 5 * GiB)
    ws = BASE + 100 * GiB
    if case == "w_overlaps_m":
        a["M"] = a["W"] + 1024
    elif case == "w_overlaps_other_g":
        b["G"] = a["W"] + 4096
    elif case == "m_overlaps_other_w":
        b["M"] = a["W"]
    elif case == "update_overlaps_g":
        a["update_out"] = a["G"] + 64
    elif case == "workspace_overlaps_w":
        ws = a["W"] + 128
    elif case == "same_w_twice":
        b["W"] = a["W"]
    descs = [mo.descriptor(64, 96, **a), mo.descriptor(64, 96, **b)]
    assert step(descs, ws=ws) == ALIAS


def test_adamw_argument_checks():
    lib = mo.load_library()
    p, g, m, v = (ctypes.c_void_p(BASE + i * GiB) for i in range(4))
    call = lambda n=100, step=1, lr=1e-3, pp=p, gg=g, mm=m, vv=v: lib.adamw_tail_step(
        pp, gg, mm, vv, n, step, lr, 0.9, 0.999, 1e-8, 0.01, None)
    assert call(n=0) == OK
    assert call(n=-1) == INVALID
    assert call(step=0) == INVALID
    assert call(lr=math.nan) == INVALID
    assert call(pp=ctypes.c_void_p(0)) == INVALID
    assert call(vv=ctypes.c_void_p(BASE + 16)) == ALIAS


def test_copy_and_worklist_argument_checks():
    lib = mo.load_library()
    assert lib.mo_device_copy(ctypes.c_void_p(BASE), ctypes.c_void_p(BASE + GiB), 15, None) == INVALID
    assert lib.mo_device_copy(ctypes.c_void_p(BASE + 8), ctypes.c_void_p(BASE + GiB), 16, None) == INVALID
    assert lib.mo_device_copy(ctypes.c_void_p(BASE), ctypes.c_void_p(BASE + 16), 64, None) == ALIAS
    assert lib.mo_device_copy(ctypes.c_void_p(BASE), ctypes.c_void_p(BASE + GiB), 0, None) == OK
    arr, n = B._array([desc()])
    size = ctypes.c_size_t(0)
    hp = mo.hparams()
    assert lib.muon_build_worklist(arr, n, ctypes.byref(hp), None, ctypes.byref(size)) == OK
    small = ctypes.c_size_t(size.value - 1)
    buf = ctypes.create_string_buffer(size.value)
    assert lib.muon_build_worklist(arr, n, ctypes.byref(hp), buf, ctypes.byref(small)) == INVALID
    assert lib.muon_build_worklist(arr, n, ctypes.byref(hp), buf, None) == INVALID
    assert lib.muon_workspace_bytes(arr, n, ctypes.byref(hp), None) == INVALID


def test_phase_list_matches_header():
    text = open(HEADER).read()
    ids = {m.group(1).lower(): int(m.group(2))
           for m in re.finditer(r"#define MO_PHASE_(\w+)\s+(\d+)", text)}
    assert ids.pop("count") == len(B.PHASES)
    for name, i in ids.items():
        assert B.PHASES[i] == name


def test_profile_read_empty():
    ms = (ctypes.c_double * len(B.PHASES))()
    cnt = (ctypes.c_int64 * len(B.PHASES))()
    lib = mo.load_library()
    assert lib.mo_profile_read(ms, cnt) == OK
    assert lib.mo_profile_read(None, cnt) == INVALID
    assert sum(cnt) == 0


def test_planning_limits_fail_fast():
    """Sizes whose work list would not fit host memory are refused before any
    planning (the size query returns at once)."""
    import time
    t0 = time.perf_counter()
    with pytest.raises(mo.MoError):
        mo.workspace_bytes([desc(1 << 23, 1 << 23)], mo.hparams())
    many = [desc(1 << 17, 1 << 17, k=k) for k in range(300)]  # 300 x 2^18 tiles > 2^26
    with pytest.raises(mo.MoError):
        mo.workspace_bytes(many, mo.hparams())
    assert time.perf_counter() - t0 < 5


def test_noalloc_entry_point_checks_without_hip():
    """The allocation-free step validates like muon_owner_step and refuses a
    bucket beyond its static array before touching the device."""
    lib = mo.load_library()
    hp = mo.hparams()
    assert lib.muon_owner_step_noalloc(None, 0, ctypes.byref(hp), None) == OK
    assert lib.muon_owner_step_noalloc(None, 1, ctypes.byref(hp), None) == INVALID
    assert lib.muon_owner_step_noalloc(None, 0, None, None) == INVALID
    base = 1 << 44
    big = [mo.descriptor(8192, 8192, W=base, G=base + (1 << 34), M=base + (2 << 34))]
    arr, n = B._array(big)
    assert mo.workspace_bytes(big, hp) > mo.NOALLOC_SCRATCH_BYTES
    assert lib.muon_owner_step_noalloc(arr, n, ctypes.byref(hp), None) == WS_SMALL
    bad = [mo.descriptor(16, 16, W=base, G=0, M=base + (2 << 34))]
    arr, n = B._array(bad)
    assert lib.muon_owner_step_noalloc(arr, n, ctypes.byref(hp), None) == INVALID
