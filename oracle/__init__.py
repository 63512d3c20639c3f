"""CPU oracle for fused LM-head Gumbel sampling.

TEST INFRASTRUCTURE: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark import this package.  The product library never does, and
the two share no code.  See fs_oracle.py for the definitions and citations.
"""
