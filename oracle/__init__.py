"""Float64 CPU oracle for the Qwen3-0.6B-shape decoder forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the library, its Python binding or
its kernels may import, call or link anything in this package; only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP path: it receives the
same seeded bfloat16 bit patterns and widens them exactly to float64.
"""
from .qwen3 import *  # noqa: F401,F403
