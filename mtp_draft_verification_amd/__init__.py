"""MI355X-native verify step of MTP speculative decoding (libspecverify).

The product is the C-ABI library ``libspecverify.so`` (include/specverify.h),
built from the HIP kernels in ``csrc/`` for gfx950.  This package holds its thin
ctypes binding (``_lib``: the C entry points under the same names), a driver
that strings those calls into the verify step of a decoder stack (``step``),
the workload geometry (``configs``) and the seeded synthetic inputs
(``inputs``).  Importing the package does not load the library; the first call
does, and raises if it has not been built.
"""
from ._lib import (SvError, sv_accept, sv_embed, sv_geglu, sv_linear, sv_linear_workspace,  # noqa: F401
                   sv_lmhead_select, sv_lmhead_workspace, sv_rmsnorm, sv_status_string,
                   sv_verify_attn, sv_verify_attn_workspace, sv_version)
