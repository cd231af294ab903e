"""fp64 CPU oracle for one rank's share of context-parallel attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package.  The product path
(``sequence_attention_dits_amd``) never imports it and shares no code with it.
"""

from .oracle import (  # noqa: F401
    build,
    split_offsets,
    positions,
    zigzag_chunks,
    seq2head,
    head2seq,
    seq2head_index,
    attention,
    attention_bwd,
    lse_merge,
    ring_pass,
    uaa_pass,
    usp_pass,
    num_threads,
)
