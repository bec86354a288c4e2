"""Float64 CPU oracle for split-KV (Flash-Decoding) decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code, header, table or helper with the
HIP library in ``decode_attention_fd_amd/``; the two meet only through the
seeded tensors of ``fd_workloads``.

Contents
--------
``attention``  the definition of decode attention written out in float64,
               the attention state of a KV segment, the two exact merges
               (``(m, l, u)`` and ``(o, lse)`` forms), split partitions and
               an independent split-then-merge path.
``plan``       the wave-efficiency split-count rule of "Flash-Decoding:
               Split-KV Attention for Long-Context Decode" §6, and the
               same rule with the workspace-traffic bound of that section's
               overhead check, as the planner applies it on 256 CUs.

Pins (tests/test_oracle.py, tests/test_oracle_plan.py) tie every function to
values the pages print, closed forms, library routines (scipy's softmax and
logsumexp) or brute force. Where no pin exists the docstring says
"parity unpinned".
"""
from . import attention, plan  # noqa: F401
