"""Dobb optimizer step on MI355X (gfx950): HIP kernels behind a C ABI (libdobb.so).

The method is "Dobb: Shard-Local Preconditioning in Block-Diagonal Eigenbases" (arXiv 2610.39412):
per weight, block-diagonal input-activation second moments (EMA), a complete eigenbasis per block,
and the update sign(M_b Q_b) Q_b^T.  ``_abi`` binds the C entry points one to one; ``optimizer``
drives them with a refresh cadence, as a torch optimizer.
"""
from ._abi import (DOBB_BF16, DOBB_F32, DOBB_NORM_COL_L2, DOBB_NORM_IDENTITY, DOBB_NORM_SIGN,  # noqa: F401
                   DOBB_OP_ACCUMULATE, DOBB_OP_REFRESH, DOBB_OP_STEP, DOBB_REFRESH_EXACT,
                   DOBB_REFRESH_ORTH_ITER, DobbError, HParams, Shape, dobb_abi_version,
                   dobb_accumulate_moment, dobb_accumulate_moment_grouped, dobb_profile_enable,
                   dobb_profile_read, dobb_profile_reset, dobb_refresh_basis, dobb_refresh_basis_grouped,
                   dobb_step, dobb_step_grouped, dobb_step_noalloc, dobb_workspace_size, lib, make_hparams,
                   status_string, DOBB_ERR_WORKSPACE, DOBB_NOALLOC_SCRATCH_BYTES, DOBB_WS_BF16_BASIS,
                   DOBB_OP_STEP_G, dobb_step_g, dobb_step_g_grouped, DOBB_REFRESH_ORTH_ITER_CHOLQR)
