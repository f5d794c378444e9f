"""fp64 CPU oracle for the owner-side Muon step and the AdamW tail.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in this
package.  The HIP library and its Python binding never import it, share no code,
table or constant generator with it, and fail loudly when their own extension is
missing instead of falling back here.

Sources (cited by page title and section, never by file or line):
  [P] "MatrixFSDP: communication-free matrix optimizers under ZeRO-3 parameter
      sharding" (academ.us article 2607.05895) - the paper.
  [A] the paper's abstract excerpt on its pith.science record.

What is computed (one Muon step on every whole 2D matrix an owner holds, one
AdamW step on the packed non-2D tail):
  muon.momentum          EMA momentum + Nesterov blend           [A]; [P §5.1]
  muon.newton_schulz     Frobenius normalisation + quintic NS    [P §2]; [P §5.1]
  muon.lr_multiplier     shape-scaled learning rate              [P §5.1]
  muon.muon_step         the whole owner step on one matrix      [P §3, §4.4]
  muon.muon_bucket       the owner step over a bucket            [P §3, §4.4]
  adamw.adamw_step       decoupled-decay Adam on the tail        [P §3, §5.1]
  worklist.build         byte-exact twin of the host work list   (no page defines it)
  planner.plan/score     owner planner and its bandwidth model    [P §4.1, §4.2]
  shampoo.shampoo_step   Shampoo on the owners (coupled Newton)   [P §5.7]
  soap.soap_step         SOAP on the owners (Adam, eigenbasis)    [P §5.7]

Every function is pinned by tests under ``tests/`` against something other than
itself (SVD brute force, closed forms, invariants, library witnesses); the pins are
listed in each function's docstring.
"""
from . import adamw, muon  # noqa: F401
