"""fp64 CPU oracle for audio prefill KV-cache compression.

Test infrastructure: only tests/, the smoke check and bench.py's CPU-baseline
leg may import it.  It shares no code with the HIP library.
"""
