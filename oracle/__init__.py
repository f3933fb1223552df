"""CPU oracle of the VAR-Q packed KV-cache hot path.

TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg.  The product library never imports it.
"""
