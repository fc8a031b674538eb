"""CPU fp64 oracle for VQ-KV decode attention — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library under
``vector_quantized_bit_amd`` never imports it and shares no code with it.

See ``oracle/vq_oracle.py`` for the functions and what pins each one.
"""
from .vq_oracle import *  # noqa: F401,F403
