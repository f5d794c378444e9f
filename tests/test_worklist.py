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

from worklist_cases import ADJ, CASES, DT, fake_descs, hp_dict, parse_worklist as _parse


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


@pytest.mark.parametrize("key", list(CASES))
def test_dispatch_lists_cover_every_tile_once(key):
    """Every Gram / Poly upper-triangle tile and every Update tile is covered by
    its parts exactly once, parts have a width of 4, 2 or 1 column blocks of 64,
    and only pad entries carry the pad index."""
    descs, hp = CASES[key]
    wl, _ = c_build(descs, hp)
    recs, lists = _parse(wl)
    for phase, items in zip(("gram", "poly", "update"), lists):
        assert len(items) % 8 == 0
        cover = {}
        for mat, ti, tj, nb in items:
            if mat == 0xFFFFFFFF:
                assert (ti, tj, nb) == (0, 0, 0)
                continue
            assert nb in (1, 2, 4)
            c0 = 64 * nb * tj
            m_pad, n_pad = recs[mat]
            width = m_pad if phase != "update" else n_pad
            assert 256 * ti < m_pad and c0 + 64 * nb <= width
            for c in range(c0 // 64, c0 // 64 + nb):
                keyc = (mat, ti, c)
                assert keyc not in cover, (phase, keyc)
                cover[keyc] = True
        want = set()
        for mat, (m_pad, n_pad) in enumerate(recs):
            tm = m_pad // 256
            for ti in range(tm):
                if phase == "update":
                    cols = range(n_pad // 64)
                else:
                    cols = [c for tj in range(ti, tm) for c in range(4 * tj, 4 * tj + 4)]
                want.update((mat, ti, c) for c in cols)
        assert set(cover) == want, phase


def test_underfilled_launch_uses_narrow_tiles():
    """A bucket with few tiles per XCD queue splits them (quarter width when the
    parts still fit the XCD's 32 CUs).  In the decoder-layer bucket the Update
    queues (98 tiles each) split only the 2 tiles of their last round, the Poly
    queues (31-32 tiles) none, and the Gram queues that the K-length balance
    left short (the long-K tiles) split all of theirs."""
    descs, hp = CASES["ragged_not_tile_multiple"]
    _, lists = _parse(c_build(descs, hp)[0])
    for items in lists:
        assert {nb for m, _, _, nb in items if m != 0xFFFFFFFF} == {1}
    descs, hp = CASES["decoder_layer_h2048"]
    _, lists = _parse(c_build(descs, hp)[0])
    upd = [nb for m, _, _, nb in lists[2] if m != 0xFFFFFFFF]
    assert upd.count(4) == 768 and upd.count(1) == 64 and len(upd) == 832
    assert {nb for m, _, _, nb in lists[1] if m != 0xFFFFFFFF} == {4}
    gram = [(m, nb) for m, _, _, nb in lists[0] if m != 0xFFFFFFFF]
    assert {nb for _, nb in gram} == {1, 2, 4}
