"""CPU oracle for the W8A8 INT8 Linear path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this package imports nothing from the product path.

Every function is a plain, slow, obviously correct numpy implementation of one
step of the method, citing the passage it follows. See ``w8a8_oracle`` for the
steps and the readings taken where the pages are silent.
"""
from .w8a8_oracle import *  # noqa: F401,F403
from .w8a8_oracle import __all__  # noqa: F401
