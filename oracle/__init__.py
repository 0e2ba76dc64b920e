"""CPU oracle for the FAST-AR attention step (TEST INFRASTRUCTURE ONLY).

Plain, slow, fp64 NumPy code that states what each stage of the step computes,
taken from the FAST-AR pages (see ``fastar_oracle``'s header for the passages).
It exists to check the HIP library, never to stand in for it: only the tests,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may import it.
It imports nothing from the HIP package and the HIP package imports nothing
from it; the only code the two share is the seeded input generator
(``workloads``), which holds no part of the method's arithmetic.

Parity status of each function is listed in ``fastar_oracle``'s header.
"""
from .fastar_oracle import (  # noqa: F401
    TIE_EPS, ann_hash, ann_quantize, bucket_sort, key_context, key_counts, annsa, annsa_multi, bucket_fields, annca,
    tempcache_top1, tempcache_commit, tempcache_update, eviction_candidates, attention_step,
)
