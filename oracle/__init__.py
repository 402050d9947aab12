"""CPU oracle for the HCA / CSA / SWA hybrid sparse attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (``sparse_hybrid_attention_amd``) and imports nothing from it.

Everything is plain NumPy in float64.  See ``hybrid_oracle.py`` for the
functions, the passages of the source pages each follows, and the readings
taken where those pages are silent.
"""
from .hybrid_oracle import *  # noqa: F401,F403
