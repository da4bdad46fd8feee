"""CPU oracle for the MoE expert-MLP path -- test infrastructure only.

Importable only from ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; the GPU library never uses it.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
