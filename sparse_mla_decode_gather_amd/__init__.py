"""MI355X-native sparse MLA decode with an index-driven KV gather.

The compute path lives in ``libsparsemla.so`` (hand-written HIP for gfx950
behind a C ABI, ``include/sparsemla.h``).  ``sparse_mla_decode_gather_amd.lib``
is a thin ctypes binding with the same entry-point names; it only marshals
arguments.  ``workloads`` draws the seeded synthetic inputs.
"""

__all__ = ["lib", "workloads"]
