"""fp64 CPU oracle for paged MLA latent decode.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow definition of what
the HIP path computes; it exists to check that path.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library (``paged_mla_latent_amd``)
and imports nothing from it; both sides take their inputs from ``workloads``.

Contents
--------
numerics : bf16 and OCP e4m3fn formats; per-128-value block quantisation.
mla      : slot addressing, row decoding, attention over gathered rows (with and
           without the rotary part; through a block table or per-query index lists),
           log-sum-exp merge of partitions, the cache-row packing, and the context
           gather with fp8 -> bf16 upconvert.

Every function is pinned by ``tests/test_oracle.py`` against brute force,
closed forms, invariants and library routines.  Parity pins for each function
are listed at the top of that test file.
"""
from .numerics import (E4M3_MAX, E4M3_TABLE, bf16_to_f32, bf16_to_f64, e4m3_decode,
                       e4m3_encode, f32_to_bf16_bits, quantize_block128)
from .mla import (LATENT, ROPE, ROW, ROW_BYTES, attend, attend_kv, cache_write, decode, decode_gla2, decode_mtp, decode_nope, decode_sparse,
                  decode_rank,
                  element_offset, element_offset_int32, gather_context, gather_rows, gather_rows_fast,
                  merge, pack_rows, rows_from_bytes, slot_of, split_ranges, upconvert_rows)

__all__ = [
    "E4M3_MAX", "E4M3_TABLE", "bf16_to_f32", "bf16_to_f64", "e4m3_decode", "e4m3_encode", "f32_to_bf16_bits", "gather_context", "upconvert_rows",
    "quantize_block128", "LATENT", "ROPE", "ROW", "ROW_BYTES", "attend", "cache_write",
    "decode", "decode_mtp", "decode_nope", "decode_sparse", "attend_kv", "decode_gla2", "decode_rank", "element_offset", "element_offset_int32", "gather_rows", "gather_rows_fast",
    "merge", "pack_rows", "rows_from_bytes", "slot_of", "split_ranges",
]
