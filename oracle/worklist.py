"""Independent Python builder of the host work list (test infrastructure).

The work list is this library's own data structure (no page defines it); its
byte layout is specified in ``include/mo.h`` (muon_build_worklist) and the
record comments there.  This twin is written from that specification with
Python's ``struct`` so that the C++ builder can be checked byte for byte.

Layout (little-endian, natural alignment, version 5):
  header (128 B): magic 'MOWL', version, n_mats, ns_steps, ns_dtype, gemm_tile,
      mom_tile, elem_bytes, n_mom_items, n_gram_items, n_poly_items,
      n_upd_items, max_partials, gemm_waves, mats_offset, gram_offset, poly_offset,
      upd_offset, wl_bytes, ws_bytes (u64), ns_a, ns_b, ns_c, eps (f32), 2 x 0
  matrix record (192 B) per non-empty descriptor, descriptor order: W, G, M,
      update_out (u64), ld_w, ld_g, ld_m, ld_u (i64; 0 -> cols), off_X,
      off_Xt0, off_Xt1, off_A, off_B, off_partials, off_scale (u64), rows,
      cols, m, n, m_pad, n_pad, flags, desc_index, mom_begin, mom_tiles_c,
      n_partials (u32), lr_eff, decay (f32), 5 x 0
  items (16 B: u32 matrix record index, tile row ti, tile column tj, width
      nb; the tile covers rows 256 ti .. +256 and columns 64 nb tj .. +64 nb):
      Gram, Poly, Update dispatch lists (entry b is run by workgroup b), each
      256-byte aligned and a multiple of 8 long; see dispatch() below
Workspace regions follow the list, per record: X, Xt0, Xt1 (m_pad*n_pad
elements each), A, B (m_pad^2), partials (n_partials fp32), scale (16 B); every
region 256-byte aligned.
"""
from __future__ import annotations

import math
import struct
from typing import List, Sequence

T = 256       # GEMM tile edge
MT = 64       # momentum tile edge
ALIGN = 256
MAGIC = 0x4C574F4D

F32, BF16 = 0, 1
LR_ORIGINAL, LR_MATCH, LR_NONE = 0, 1, 2

FLAG_TRANSPOSED, FLAG_HAS_UPDATE, FLAG_W_BF16, FLAG_G_BF16 = 1, 2, 4, 8


def _up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def _f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def build(descs: Sequence[dict], hp: dict) -> bytes:
    """descs: dicts with rows, cols, W, G, M, update_out (ints), ld_w, ld_g, ld_m,
    ld_u, w_dtype, g_dtype.  hp: lr, weight_decay, ns_steps, ns_a, ns_b, ns_c,
    eps, lr_adjust, ns_dtype (ints for the enums)."""
    es = 2 if hp["ns_dtype"] == BF16 else 4
    lr = _f32(hp["lr"])
    wd = _f32(hp["weight_decay"])
    recs = []
    mom = 0
    max_partials = 0
    for i, d in enumerate(descs):
        rows, cols = d["rows"], d["cols"]
        if rows == 0 or cols == 0:
            continue
        tr = rows > cols
        m, n = min(rows, cols), max(rows, cols)
        m_pad, n_pad = _up(m, T), _up(n, T)
        r_pad, c_pad = (n_pad, m_pad) if tr else (m_pad, n_pad)
        n_part = (r_pad // MT) * (c_pad // MT)
        if hp["lr_adjust"] == LR_ORIGINAL:
            factor = math.sqrt(max(1.0, rows / cols))
        elif hp["lr_adjust"] == LR_MATCH:
            factor = 0.2 * math.sqrt(float(max(rows, cols)))
        else:
            factor = 1.0
        flags = (FLAG_TRANSPOSED if tr else 0) | (FLAG_HAS_UPDATE if d.get("update_out") else 0) \
            | (FLAG_W_BF16 if d["w_dtype"] == BF16 else 0) | (FLAG_G_BF16 if d["g_dtype"] == BF16 else 0)
        recs.append(dict(W=d.get("W", 0), G=d.get("G", 0), M=d.get("M", 0), U=d.get("update_out", 0) or 0,
                         ld_w=d.get("ld_w", 0) or cols, ld_g=d.get("ld_g", 0) or cols,
                         ld_m=d.get("ld_m", 0) or cols, ld_u=d.get("ld_u", 0) or cols,
                         rows=rows, cols=cols, m=m, n=n, m_pad=m_pad, n_pad=n_pad, flags=flags,
                         desc_index=i, mom_begin=mom, mom_tiles_c=c_pad // MT, n_partials=n_part,
                         lr_eff=lr * factor, decay=1.0 - lr * wd))
        mom += n_part
        max_partials = max(max_partials, n_part)

    def ordered(work):
        idx = list(range(len(recs)))
        return sorted(idx, key=lambda j: -work(recs[j]))   # stable: ties keep order

    def upper(r):
        t = r["m_pad"] // T
        return t * (t + 1) // 2

    PAD = 0xFFFFFFFF

    def dispatch(mat_order, upper_only, k_is_n):
        """Super-blocks of 4 tile-rows x 8 tile-columns (row-major, tiles
        row-major inside), in matrix order, each costing K-length per tile.  A
        block goes to the least-loaded of 8 queues (ties: lowest); if that
        queue is under target = ceil(total / 8), it takes only
        max(1, ceil((target - load) / K-length)) tiles and the rest of the block
        goes on to the next least-loaded queue.  The list interleaves the queues
        (entry 8 j + x = j-th tile of queue x, or a pad entry)."""
        blocks = []
        for j in mat_order:
            r = recs[j]
            tm = r["m_pad"] // T
            tn = tm if upper_only else r["n_pad"] // T
            klen = r["n_pad"] if k_is_n else r["m_pad"]
            for bi in range(0, tm, 4):
                for bj in range(0, tn, 8):
                    blk = [(j, a, b, 4) for a in range(bi, min(bi + 4, tm))
                           for b in range(bj, min(bj + 8, tn)) if not upper_only or a <= b]
                    if blk:
                        blocks.append((blk, klen))
        total = sum(len(b) * k for b, k in blocks)
        target = (total + 7) // 8
        queues = [[] for _ in range(8)]
        load = [0] * 8
        for blk, klen in blocks:
            i = 0
            while i < len(blk):
                x = min(range(8), key=lambda y: (load[y], y))
                take = len(blk) - i
                if load[x] < target:
                    fit = (target - load[x] + klen - 1) // klen
                    take = min(take, max(1, fit))
                queues[x] += blk[i:i + take]
                load[x] += klen * take
                i += take
        # Queues of at most 32 tiles (32 CUs per XCD) have every tile split,
        # longer ones the len % 32 tiles of the last round: into S = 2
        # half-width tiles when 2 * (tiles split) <= 32 (S = 4 quarter widths
        # only for lists built for 4-wavefront kernels, max_split 4).
        for x, q in enumerate(queues):
            n = len(q)
            if n == 0:
                continue
            first = 0 if n <= 32 else n - n % 32
            r = n - first
            S = (1 if r == 0 else 4 if (max_split >= 4 and 4 * r <= 32)
                 else 2 if (max_split >= 2 and 2 * r <= 32) else 1)
            if S > 1:
                queues[x] = q[:first] + [(j, a, b * S + p, 4 // S) for (j, a, b, _) in q[first:]
                                         for p in range(S)]
        longest = max((len(q) for q in queues), default=0)
        return [queues[x][j] if j < len(queues[x]) else (PAD, 0, 0, 0)
                for j in range(longest) for x in range(8)]

    waves = 8 if hp["ns_dtype"] == 1 else 4   # bf16 lists: 8-wavefront kernels
    max_split = 2 if waves == 8 else 4
    gram = dispatch(ordered(lambda r: upper(r) * r["n_pad"]), True, True)
    poly = dispatch(ordered(lambda r: upper(r) * r["m_pad"]), True, False)
    upd = dispatch(ordered(lambda r: (r["m_pad"] // T) * (r["n_pad"] // T) * r["m_pad"]), False, False)

    mats_off = 128
    gram_off = _up(mats_off + 192 * len(recs), ALIGN)
    poly_off = _up(gram_off + 16 * len(gram), ALIGN)
    upd_off = _up(poly_off + 16 * len(poly), ALIGN)
    wl_bytes = _up(upd_off + 16 * len(upd), ALIGN)

    off = wl_bytes
    for r in recs:
        mn, mm = r["m_pad"] * r["n_pad"], r["m_pad"] * r["m_pad"]
        for key, size in (("off_X", mn * es), ("off_Xt0", mn * es), ("off_Xt1", mn * es),
                          ("off_A", mm * es), ("off_B", mm * es),
                          ("off_partials", r["n_partials"] * 4), ("off_scale", 16)):
            r[key] = off
            off = _up(off + size, ALIGN)
    ws_bytes = off

    out = bytearray(wl_bytes)
    struct.pack_into("<14I6Q4f2I", out, 0, MAGIC, 5, len(recs), hp["ns_steps"], hp["ns_dtype"],
                     T, MT, es, mom, len(gram), len(poly), len(upd), max_partials, waves,
                     mats_off, gram_off, poly_off, upd_off, wl_bytes, ws_bytes,
                     hp["ns_a"], hp["ns_b"], hp["ns_c"], hp["eps"], 0, 0)
    for k, r in enumerate(recs):
        struct.pack_into("<4Q4q7Q11I2f5I", out, mats_off + 192 * k,
                         r["W"], r["G"], r["M"], r["U"], r["ld_w"], r["ld_g"], r["ld_m"], r["ld_u"],
                         r["off_X"], r["off_Xt0"], r["off_Xt1"], r["off_A"], r["off_B"],
                         r["off_partials"], r["off_scale"],
                         r["rows"], r["cols"], r["m"], r["n"], r["m_pad"], r["n_pad"], r["flags"],
                         r["desc_index"], r["mom_begin"], r["mom_tiles_c"], r["n_partials"],
                         r["lr_eff"], r["decay"], 0, 0, 0, 0, 0)
    for base, items in ((gram_off, gram), (poly_off, poly), (upd_off, upd)):
        for k, item in enumerate(items):
            struct.pack_into("<4I", out, base + 16 * k, *item)
    return bytes(out)


def workspace_bytes(descs: Sequence[dict], hp: dict) -> int:
    wl = build(descs, hp)
    return struct.unpack_from("<Q", wl, 96)[0] + ALIGN
