"""Oracle package -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct CPU implementations of what the GEMM path
computes (``gemm_ref``) and of the tile-selection rules (``select_ref``).
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything here; the library itself never does, and
nothing here imports the library.
"""
