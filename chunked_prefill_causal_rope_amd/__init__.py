"""MI355X (gfx950) causal grouped-query attention with RoPE over a head-major
KV cache: a C-ABI HIP library (libattn.so, include/attn.h) and its thin
Python binding.

  api       -- ctypes binding of the C ABI (marshalling only)
  runner    -- the chunk loop and the decode step, issuing library calls
  workloads -- the workload table and seeded synthetic inputs
  build     -- in-tree hipcc build of libattn.so for gfx950
"""
from . import api, workloads  # noqa: F401
from .api import (AttnError, Batch, decode, decode_workspace_bytes, kv_append,  # noqa: F401
                  prefill_chunk, prefill_workspace_bytes, rope_apply, rope_inv_freq,
                  yarn_inv_freq)

__version__ = "0.1.0"
