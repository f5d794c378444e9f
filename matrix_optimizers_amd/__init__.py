"""MI355X-native (gfx950) owner-side Muon step, AdamW tail, Shampoo and SOAP steps.

Under owner-shaped ZeRO-3 placement ("MatrixFSDP: communication-free matrix
optimizers under ZeRO-3 parameter sharding", §3) each 2D weight is whole on one
owner, so that owner runs Muon locally on its whole matrices and AdamW on its
packed non-2D tail.  This package is that step: hand-written HIP kernels behind
the C ABI in ``include/mo.h`` (``libmo.so``), with this thin ctypes binding.

    from matrix_optimizers_amd import muon_owner_step, adamw_tail_step
    muon_owner_step([(W, G, M), ...], lr=0.02, weight_decay=0.01)
    adamw_tail_step(p, g, m, v, step=10)
    shampoo_owner_step([(W, G, L, R), ...], lr=1e-3, root_iters=20)
    soap_owner_step([(W, G, L, R, M, V), ...], lr=1e-3, step=t)

The library is loaded on first use; if it has not been built
(``python -m matrix_optimizers_amd.build``) every entry point raises.
"""
from ._binding import (  # noqa: F401
    PLAN_POLICIES, ROLE_MATRIX, ROLE_TAIL, MoError, MoMatrix, MoMuonHParams, MoRole, MuonOwnerStep,
    MoShampooHParams, MoShampooMatrix, ShampooOwnerStep, shampoo_descriptor, shampoo_hparams,
    shampoo_owner_step, shampoo_tensor_descriptor, shampoo_workspace_bytes,
    MoSoapHParams, MoSoapMatrix, SoapOwnerStep, soap_descriptor, soap_hparams, soap_owner_step,
    soap_converged, soap_tensor_descriptor, soap_workspace_bytes,
    PHASES, adamw_tail_step, build_worklist, descriptor, device_copy, hparams, load_library,
    mo_status_string, muon_build_worklist, muon_owner_step, muon_owner_step_noalloc, muon_workspace_bytes,
    NOALLOC_SCRATCH_BYTES, plan_layout,
    plan_owners, plan_score, profile_enable, profile_read, status_string, tensor_descriptor,
    workspace_bytes,
)
