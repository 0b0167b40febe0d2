"""CPU oracle for paged MLA decode — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy (fp64) definitions of what the HIP path
computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import anything from here; the product path
(``long_context_mla_amd``) never does, and shares no code with it.

Modules
-------
``e4m3``      OCP E4M3FN decode table and round-to-nearest-even saturating encoder.
``mla``       attention definition (``decode_ref``), per-row split partials
              (``partial_ref``), the log-sum-exp merge (``merge_ref``) and the
              FP8 cache append (``append_ref``), plus a pure-Python loop version
              of the attention (``decode_naive``) for tiny cases.
``integrity`` the KV page-tag check (``check_pages_ref``): per-request status
              bits and the lengths decode may use.

Parity pins for every function live in ``tests/test_oracle_*.py``; none of the
oracle's functions is left unpinned.
"""

from . import e4m3, integrity, mla  # noqa: F401
