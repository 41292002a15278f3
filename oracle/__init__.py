"""fp64 CPU oracle for MLA paged-KV decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything from here.  The
GPU library (``paged_kv_mla_req_amd``) never imports, links or calls it, and
this package shares no code with it: the only thing both sides use is the
seeded input generator in ``workloads/``, which contains none of the method's
arithmetic.

Every function here is pinned by ``tests/test_oracle_*.py`` against something
other than itself (a pure-Python brute force, torch's dtype casts, closed
forms and invariants).  No function is "parity unpinned".
"""

from .paged_mla import (  # noqa: F401
    PAGE_SIZE,
    V_DIM,
    bf16_to_f64,
    e4m3fn_to_f64,
    block_table,
    request_keys,
    attend,
    paged_decode,
    paged_decode_q8,
    merge_states,
)
from .kv_append import e4m3fn_encode, quantize_rows, quantize_q, set_kv_buffer  # noqa: F401
from .plan import (  # noqa: F401
    plan_reference, check_plan, plan_overhead, plan_fixed, check_fixed_plan, plan_fixed_packed,
    check_fixed_packed_plan)
