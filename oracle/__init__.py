"""ORACLE package -- test infrastructure only.

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` and by nothing else.  It shares no code with the HIP library.
"""
