"""fp64 CPU oracle of the DCP partial-merge path -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP library and never imports it.
"""
