"""CPU oracle for the HySparse2 Cross-Decoder hot path: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
anything under this directory; the product path never does.
"""
