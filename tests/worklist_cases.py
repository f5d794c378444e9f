"""Work-list test cases: the workloads and the edge cases, as descriptors with
made-up addresses.  No library or binding import (the golden-digest script uses
this with the Python twin only)."""
import struct

from matrix_optimizers_amd import workloads as wlmod

DT = {"f32": 0, "bf16": 1}
ADJ = {"original": 0, "match_rms_adamw": 1, "none": 2}


def fake_descs(shapes, w_dtype="bf16", g_dtype="bf16", with_update=False):
    """Descriptors with made-up, non-overlapping addresses (never dereferenced)."""
    out = []
    base = 1 << 40
    for i, (r, c) in enumerate(shapes):
        d = dict(rows=r, cols=c, W=base + 4 * i * (1 << 34), G=base + (4 * i + 1) * (1 << 34),
                 M=base + (4 * i + 2) * (1 << 34),
                 update_out=(base + (4 * i + 3) * (1 << 34)) if with_update else 0,
                 ld_w=0, ld_g=0, ld_m=0, ld_u=0, w_dtype=DT[w_dtype], g_dtype=DT[g_dtype])
        out.append(d)
    return out


def hp_dict(hp: wlmod.MuonHP):
    return dict(lr=hp.lr, weight_decay=hp.weight_decay, ns_steps=hp.ns_steps, ns_a=hp.ns_a,
                ns_b=hp.ns_b, ns_c=hp.ns_c, eps=hp.eps, lr_adjust=ADJ[hp.lr_adjust],
                ns_dtype=DT[hp.ns_dtype])


def workload_case(key):
    wl = wlmod.get(key)
    return fake_descs([(s.rows, s.cols) for s in wl.matrices], wl.w_dtype, wl.g_dtype), wl.hp


EDGE_CASES = {
    "one_by_one": ([(1, 1)], wlmod.MuonHP()),
    "row_and_column": ([(1, 1000), (1000, 1)], wlmod.MuonHP()),
    "empty_descriptors": ([(0, 5), (7, 0), (33, 17), (0, 0)], wlmod.MuonHP()),
    "ragged_not_tile_multiple": ([(129, 257), (300, 1000), (1000, 300)], wlmod.MuonHP(ns_dtype="f32")),
    "over_65k_update_tiles": ([(256, 8388608)], wlmod.MuonHP()),
    "match_rms_two_steps": ([(4096, 16384), (16384, 4096)],
                            wlmod.MuonHP(ns_steps=2, lr_adjust="match_rms_adamw", lr=1e-3)),
    "no_lr_adjust_zero_steps": ([(300, 200)], wlmod.MuonHP(ns_steps=0, lr_adjust="none")),
    "equal_work_ties": ([(512, 512)] * 5, wlmod.MuonHP()),
}


def all_cases():
    cases = {k: workload_case(k) for k in wlmod.WORKLOAD_ORDER + ["paper_owner_share"]}
    for k, (shapes, hp) in EDGE_CASES.items():
        cases[k] = (fake_descs(shapes, with_update=(k == "ragged_not_tile_multiple")), hp)
    return cases


CASES = all_cases()


def parse_worklist(wl: bytes):
    """Header fields, matrix records (m_pad, n_pad) and the three item lists."""
    hdr = struct.unpack_from("<14I6Q4f2I", wl, 0)
    n_mats = hdr[2]
    counts = hdr[9:12]
    mats_off, offs = hdr[14], hdr[15:18]
    recs = []
    for k in range(n_mats):
        rec = struct.unpack_from("<4Q4q7Q11I2f5I", wl, mats_off + 192 * k)
        recs.append((rec[19], rec[20]))   # m_pad, n_pad
    lists = [[struct.unpack_from("<4I", wl, off + 16 * i) for i in range(cnt)]
             for off, cnt in zip(offs, counts)]
    return recs, lists
