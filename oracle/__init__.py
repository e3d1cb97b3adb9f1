"""CPU oracle for the InternVL visual-token compression connector.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library.  It is
plain numpy in float64 and shares no code with ``vlm_visual_token_amd``.
"""
from .connector import *  # noqa: F401,F403
from . import connector  # noqa: F401
