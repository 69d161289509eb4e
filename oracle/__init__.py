"""fp64 CPU oracle for the KDA forward pass.

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  It shares no code
with the HIP path (chunked_gated_delta_amd) and neither imports the other.
"""
