"""CPU oracle for paged KV-cache attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path
(``paged_kv_cache_67_amd``) never imports it and shares no code with it; the
two meet only in the seeded inputs of ``workloads``.

Every function here is the plain, slow definition of what the path computes,
in float64, with the sources it follows cited in its docstring.  Parity status
of each function (what pins it) is listed in ``oracle.paged_attention``.
"""

from .paged_attention import (  # noqa: F401
    copy_blocks,
    decode,
    decode_partials,
    gather_rows,
    lse_merge,
    prefill,
    slot_mapping,
    store_kv,
    to_f64,
)
