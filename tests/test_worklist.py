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
    """A bucket with few tiles per XCD queue splits them, into quarter widths
    when the parts still fit the XCD's 32 CUs and the list is built for the
    fp32 (4-wavefront) kernels, into half widths for the bf16 (8-wavefront)
    kernels, which have no quarter width.  The ragged case runs fp32.  In the
    bf16 decoder-layer bucket the Update queues (98 tiles each) split only the
    2 tiles of their last round, the Poly queues (31-32 tiles) none, and the
    Gram queues that the K-length balance left short (the long-K tiles) split
    theirs."""
    descs, hp = CASES["ragged_not_tile_multiple"]
    _, lists = _parse(c_build(descs, hp)[0])
    for items in lists:
        assert {nb for m, _, _, nb in items if m != 0xFFFFFFFF} == {1}
    descs, hp = CASES["decoder_layer_h2048"]
    _, lists = _parse(c_build(descs, hp)[0])
    upd = [nb for m, _, _, nb in lists[2] if m != 0xFFFFFFFF]
    assert upd.count(4) == 768 and upd.count(2) == 32 and len(upd) == 800
    assert {nb for m, _, _, nb in lists[1] if m != 0xFFFFFFFF} == {4}
    gram = [(m, nb) for m, _, _, nb in lists[0] if m != 0xFFFFFFFF]
    assert {nb for _, nb in gram} == {2, 4}


# ---- record-level pins, derived from the step's definition (not from the twin) ----

import math

import numpy as np

from oracle import muon as omuon

HDR_FMT = "<14I6Q4f2I"
REC_FMT = "<4Q4q7Q11I2f5I"
REC_FIELDS = ("W G M U ld_w ld_g ld_m ld_u off_X off_Xt0 off_Xt1 off_A off_B off_partials off_scale "
              "rows cols m n m_pad n_pad flags desc_index mom_begin mom_tiles_c n_partials lr_eff decay "
              "r0 r1 r2 r3 r4").split()
HDR_FIELDS = ("magic version n_mats ns_steps ns_dtype gemm_tile mom_tile elem_bytes n_mom n_gram n_poly "
              "n_upd max_partials res0 mats_offset gram_offset poly_offset upd_offset wl_bytes ws_bytes "
              "ns_a ns_b ns_c eps res1 res2").split()


def full_parse(wl: bytes):
    import struct
    h = dict(zip(HDR_FIELDS, struct.unpack_from(HDR_FMT, wl, 0)))
    recs = [dict(zip(REC_FIELDS, struct.unpack_from(REC_FMT, wl, h["mats_offset"] + 192 * k)))
            for k in range(h["n_mats"])]
    return h, recs


def f32(x):
    return float(np.float32(x))


@pytest.mark.parametrize("key", list(CASES))
def test_records_follow_the_step_definition(key):
    """Each record against what the step fixes, computed here from the
    descriptor and hyperparameters alone:
      * the Gram side is the short side: transposed iff rows > cols, m = min,
        n = max, both padded with zeros to the 256 GEMM tile;
      * lr_eff is fp32(fp32(lr) x the shape factor of the lr adjustment, in
        fp64), with the factor taken from the oracle's definition; the decay
        is fp32(1 - fp32(lr) fp32(wd));
      * descriptor fields (pointers, strides with 0 meaning cols, dtypes)
        are carried over, empty descriptors are dropped, order is kept;
      * momentum tiles: 64 x 64 tiles of the weight's padded frame, numbered
        matrix after matrix;
      * every workspace region is 256-byte aligned, lies after the list and
        inside ws_bytes, and no two regions overlap; the reported workspace
        size is ws_bytes plus 256 bytes of alignment slack."""
    descs, hp = CASES[key]
    wl, ws = c_build(descs, hp)
    h, recs = full_parse(wl)
    live = [(i, d) for i, d in enumerate(descs) if d["rows"] and d["cols"]]
    es = 2 if hp.ns_dtype == "bf16" else 4
    assert h["magic"] == 0x4C574F4D and h["n_mats"] == len(live)
    assert (h["gemm_tile"], h["mom_tile"], h["elem_bytes"]) == (256, 64, es)
    assert h["ns_steps"] == hp.ns_steps and h["ns_dtype"] == DT[hp.ns_dtype]
    assert (h["ns_a"], h["ns_b"], h["ns_c"], h["eps"]) == (f32(hp.ns_a), f32(hp.ns_b), f32(hp.ns_c),
                                                           f32(hp.eps))
    assert h["wl_bytes"] == len(wl) and len(wl) % 256 == 0
    assert ws == h["ws_bytes"] + 256
    pad = lambda x: -(-x // 256) * 256
    regions = [(0, h["wl_bytes"])]
    mom = 0
    for (i, d), r in zip(live, recs):
        rows, cols = d["rows"], d["cols"]
        tr = rows > cols
        m, n = min(rows, cols), max(rows, cols)
        assert (r["rows"], r["cols"], r["m"], r["n"]) == (rows, cols, m, n)
        assert (r["m_pad"], r["n_pad"]) == (pad(m), pad(n))
        assert bool(r["flags"] & 1) == tr
        assert bool(r["flags"] & 2) == bool(d["update_out"])
        assert bool(r["flags"] & 4) == (d["w_dtype"] == DT["bf16"])
        assert bool(r["flags"] & 8) == (d["g_dtype"] == DT["bf16"])
        assert r["desc_index"] == i
        assert (r["W"], r["G"], r["M"], r["U"]) == (d["W"], d["G"], d["M"], d["update_out"])
        for f in ("ld_w", "ld_g", "ld_m", "ld_u"):
            assert r[f] == (d[f] or cols)
        lr32 = np.float64(np.float32(hp.lr))
        want_lr = np.float32(lr32 * omuon.lr_multiplier(rows, cols, hp.lr_adjust))
        assert np.float32(r["lr_eff"]) == want_lr, (r["lr_eff"], want_lr)
        want_decay = np.float32(1.0 - lr32 * np.float64(np.float32(hp.weight_decay)))
        assert np.float32(r["decay"]) == want_decay
        # momentum tiles over the weight's own frame, padded to 256
        r_pad, c_pad = (pad(n), pad(m)) if tr else (pad(m), pad(n))
        assert r["mom_tiles_c"] == c_pad // 64
        assert r["n_partials"] == (r_pad // 64) * (c_pad // 64)
        assert r["mom_begin"] == mom
        mom += r["n_partials"]
        mn, mm = pad(m) * pad(n) * es, pad(m) * pad(m) * es
        for off, size in ((r["off_X"], mn), (r["off_Xt0"], mn), (r["off_Xt1"], mn), (r["off_A"], mm),
                          (r["off_B"], mm), (r["off_partials"], 4 * r["n_partials"]), (r["off_scale"], 16)):
            assert off % 256 == 0
            regions.append((off, off + size))
    assert h["n_mom"] == mom
    assert h["max_partials"] == max([r["n_partials"] for r in recs], default=0)
    regions.sort()
    for (a0, a1), (b0, b1) in zip(regions, regions[1:]):
        assert a1 <= b0, (a0, a1, b0, b1)
    assert regions[-1][1] <= h["ws_bytes"]
    # the three item lists sit inside the list, 256-aligned, in order, disjoint
    offs = [h["gram_offset"], h["poly_offset"], h["upd_offset"]]
    ends = [o + 16 * c for o, c in zip(offs, (h["n_gram"], h["n_poly"], h["n_upd"]))]
    assert all(o % 256 == 0 for o in offs)
    assert h["mats_offset"] + 192 * h["n_mats"] <= offs[0] and ends[0] <= offs[1] and ends[1] <= offs[2]
    assert ends[2] <= h["wl_bytes"]


def test_lr_factors_at_the_workload_shapes():
    """Spot values of lr_eff at the workload shapes, by hand: sqrt(5632/2048),
    sqrt(14336/4096) = sqrt(28672/8192) = sqrt(3.5), sqrt(128256/4096), 1 for
    wide and square matrices, and 0.2 sqrt(max side) for match_rms_adamw."""
    cases = [((5632, 2048), "original", math.sqrt(5632 / 2048)),
             ((2048, 5632), "original", 1.0), ((4096, 4096), "original", 1.0),
             ((28672, 8192), "original", math.sqrt(3.5)), ((14336, 4096), "original", math.sqrt(3.5)),
             ((128256, 4096), "original", math.sqrt(31.3125)),
             ((4096, 16384), "match_rms_adamw", 0.2 * 128.0), ((300, 200), "none", 1.0)]
    for (r, c), adj, factor in cases:
        hp = wlmod.MuonHP(lr_adjust=adj, lr=0.02)
        _, recs = full_parse(c_build(fake_descs([(r, c)]), hp)[0])
        want = np.float32(np.float64(np.float32(0.02)) * factor)
        assert np.float32(recs[0]["lr_eff"]) == want, (r, c, adj)
