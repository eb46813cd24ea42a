"""Float64 CPU oracle for Jet-Long bifocal RoPE attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything under
``oracle/``.  The product path (the HIP library and its Python binding)
never imports, links or calls it, and shares no code with it.

Every function is pinned by ``-m "not gpu"`` tests in ``tests/`` against
facts the pages and the mathematics fix (a worked schedule example, closed
forms, exact identities, a brute-force evaluation by a different route and a
textbook library routine).  No function here is "parity unpinned".
"""
from .jetlong_oracle import (  # noqa: F401
    group_size, alias_position, correction_offset, inv_freq, rope_rotate,
    remote_view, bifocal_attention, plain_causal_attention, decode_attention,
    inclusion_exclusion_attention, softmax_rows, fi_scale, fi_ramp, fi_inv_freq, fi_remote_view,
    bifocal_attention_fi, decode_attention_fi,
)
