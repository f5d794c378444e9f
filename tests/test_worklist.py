"""The C++ work-list builder against the independent Python twin (byte for byte)
and against committed golden digests.  CPU only: the builder is host code."""
import hashlib
import json
import os

import pytest

import matrix_optimizers_amd as mo
from matrix_optimizers_amd import workloads as wlmod
from oracle import worklist as twin

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "worklist_digests.json")

from worklist_cases import ADJ, CASES, DT, fake_descs, hp_dict


def c_build(descs, hp: wlmod.MuonHP):
    cd = [mo.descriptor(d["rows"], d["cols"], W=d["W"], G=d["G"], M=d["M"], update_out=d["update_out"],
                        w_dtype=d["w_dtype"], g_dtype=d["g_dtype"], ld_w=d["ld_w"], ld_g=d["ld_g"],
                        ld_m=d["ld_m"], ld_u=d["ld_u"]) for d in descs]
    h = mo.hparams(lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum,
                   nesterov=hp.nesterov, ns_steps=hp.ns_steps,
                   ns_coefficients=(hp.ns_a, hp.ns_b, hp.ns_c), eps=hp.eps,
                   adjust_lr_fn=hp.lr_adjust, ns_dtype=hp.ns_dtype)
    return mo.build_worklist(cd, h), mo.workspace_bytes(cd, h)


@pytest.mark.parametrize("key", list(CASES))
def test_worklist_matches_python_twin(key):
    descs, hp = CASES[key]
    got, ws = c_build(descs, hp)
    want = twin.build(descs, hp_dict(hp))
    assert len(got) == len(want)
    if got != want:
        first = next(i for i in range(len(got)) if got[i] != want[i])
        pytest.fail(f"first differing byte at {first} of {len(got)}")
    assert ws == twin.workspace_bytes(descs, hp_dict(hp))


def test_worklist_golden_digests():
    """Digests written by tests/golden/make_worklist_golden.py (which calls only
    the Python twin)."""
    golden = json.load(open(GOLDEN))
    for key, digest in golden.items():
        descs, hp = CASES[key]
        got, _ = c_build(descs, hp)
        assert hashlib.sha256(got).hexdigest() == digest, key


def test_strided_descriptor_records_strides():
    d = fake_descs([(100, 60)])
    d[0].update(ld_w=64, ld_g=72, ld_m=80, ld_u=0)
    got, _ = c_build(d, wlmod.MuonHP())
    assert got == twin.build(d, hp_dict(wlmod.MuonHP()))


def test_side_beyond_limit_is_unsupported():
    with pytest.raises(mo.MoError) as e:
        c_build(fake_descs([(1, (1 << 23) + 1)]), wlmod.MuonHP())
    assert e.value.status == -2
