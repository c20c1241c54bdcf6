"""CPU oracle for NF4 blockwise quantization and the NF4 dequant-GEMMs.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything under
``oracle/``.  The product library (``dequant_gemm_amd``) never imports it and
shares no code, constants or tables with it; the two meet only through the
seeded inputs of ``synth``.

Every function is plain numpy / Python integer arithmetic written from the
method's definition; see ``oracle/nf4_oracle.py`` for the citations.
"""
from .nf4_oracle import *  # noqa: F401,F403
