"""CPU oracle for sparse MLA decode with an index-driven KV gather.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The product path (the HIP library and its Python binding) never does, and
shares no code, header, table or helper with this package.

Everything is plain NumPy in float64 (the pages fix no precision), written
from the method's definition as the FlashInfer and vLLM pages state it:

* ``formats``  - the BF16 and OCP FP8 E4M3FN bit formats, decoded from their
  definitions, the 584-byte packed block-scaled FP8 row (a reading of the
  pages, see there), plus BF16 round-to-nearest-even for comparing rounded
  outputs.
* ``sparse_mla`` - the decode itself (selection, gather, sink-aware softmax,
  base-2 LSE), its split form and the LSE combine.
* ``brute``    - a second, independent formulation (multiset of pool rows,
  pure-Python loops, optional mpmath arithmetic) used to pin the first.
* ``index_builder`` - the combined index table built from decode metadata
  (SWA rows + local compressed positions through a block table).

Parity status of each function is stated in its docstring; every function
here is pinned by tests in ``tests/test_oracle_*.py`` except where a
docstring says "parity unpinned".
"""

from .formats import bf16_bits_to_f64, e4m3fn_bits_to_f64, decode_bits, \
    round_to_bf16, ue8m0_to_f64, packed584_to_f64, PACKED_ROW_BYTES
from .sparse_mla import (SWA_COLUMNS, active_slots, active_slots_segments,
                         active_slots_paged, decode_token, sparse_mla_decode,
                         sparse_mla_decode_segments, sparse_mla_decode_paged,
                         split_partials, combine, split_columns)
from .brute import (brute_force_decode, brute_force_decode_segments,
                    brute_force_decode_paged)
from .index_builder import build_combined_indices

__all__ = [
    "bf16_bits_to_f64", "e4m3fn_bits_to_f64", "decode_bits", "round_to_bf16",
    "ue8m0_to_f64", "packed584_to_f64", "PACKED_ROW_BYTES",
    "SWA_COLUMNS", "active_slots", "active_slots_segments",
    "active_slots_paged", "decode_token", "sparse_mla_decode",
    "sparse_mla_decode_segments", "sparse_mla_decode_paged", "split_partials",
    "combine", "split_columns", "brute_force_decode",
    "brute_force_decode_segments", "brute_force_decode_paged",
    "build_combined_indices",
]
