"""CPU oracle of the MoE expert layer: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg import it.
"""
