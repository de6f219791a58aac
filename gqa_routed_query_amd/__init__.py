"""gqa_routed_query_amd: grouped-query attention (GQA) and grouped query
experts (GQE) on AMD MI355X (gfx950).

The compute path is the HIP library ``libgqa.so`` (C ABI, ``include/gqa.h``);
this package only marshals torch tensors into its entry points:

* :func:`gqa_prefill` -- GQA prefill, q [B,h,T,d], k/v [B,g,T,d].
* :func:`gqa_decode` -- one decode step over a KV cache [B,g,T_max,d].
* :func:`gqa_decode_noalloc` -- the same step with the split partials in the
  library's static device scratch, for callers that cannot allocate.
* :func:`gqe_routed_prefill` -- GQE: top-k query-head experts per KV group
  per token, dense K/V.
* :func:`gqe_routed_decode` -- GQE routing applied to one decode step.
* :func:`gqe_router` -- the router's projection x W_r^T fused with the top-k.
* :func:`gqe_prefill_build` -- the GQE layer output: kept experts concatenated,
  their weighted-sum slot and the shared head.
* :func:`peak_hbm_read`, :func:`peak_mfma_bf16`, :func:`peak_attn_tile` --
  peak microbenchmarks (an HBM read stream, an MFMA-only loop, the prefill's
  attention tile loop on register operands), the measured peaks the path's
  rates are compared with.

torch provides device memory and the stream; every step of the computation
runs in the library's kernels. Importing the package fails loudly when the
library has not been built (``python gqa_routed_query_amd/build.py``).
"""
from ._binding import (  # noqa: F401
    GQA_BF16,
    GQA_F32,
    GqaError,
    abi_version,
    gqa_decode,
    gqa_decode_noalloc,
    gqa_decode_workspace_bytes,
    gqa_kv_cache_bytes,
    gqa_prefill,
    gqe_prefill_build,
    gqe_routed_decode,
    gqe_routed_prefill,
    gqe_router,
    gqe_workspace_bytes,
    last_error,
    lib_path,
    peak_attn_tile,
    peak_hbm_read,
    peak_mfma_bf16,
    status_string,
)
