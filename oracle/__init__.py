"""fp64 CPU oracle of the MosaicKV decode path -- TEST INFRASTRUCTURE ONLY.

Importable by tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg.
The product package never imports it.
"""
