"""CommVQ quantized-KV hot path for AMD MI355X (gfx950).

The computation lives in ``libcommvq.so`` (HIP kernels behind the C ABI in
``include/commvq.h``); ``_lib`` binds it with ctypes under the same names and
``api`` adds tensor-allocating conveniences on top. Importing the package does
not load the library; the first call does, and fails if it is not built.
"""

from . import _lib  # noqa: F401
from ._lib import (COMMVQ_OK, CommvqError, commvq_abi_version, commvq_append,  # noqa: F401
                   commvq_bits_per_scalar, commvq_code_bytes_per_token, commvq_decode_attention,
                   commvq_decode_step, commvq_decode_workspace_bytes, commvq_encode, commvq_last_error,
                   commvq_validate_codebook, make_codebook, make_rope)
