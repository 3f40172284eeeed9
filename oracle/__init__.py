"""CPU oracle for the VDN hybrid attention layer forward -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The GPU path never imports it and shares no code with it.
"""
