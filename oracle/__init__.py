"""fp64 CPU oracle for the MoE-VQ routed-expert step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library or its binding;
the only module both sides use is ``synth`` (seeded random draws, no arithmetic).

See ``oracle/moe_vq_oracle.py`` for the definitions and their sources.
"""
from .moe_vq_oracle import *  # noqa: F401,F403
