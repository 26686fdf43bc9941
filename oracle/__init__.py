"""CPU oracle of the dequant-on-use qgemv / MoE path.

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's
CPU-baseline leg import this package.  See coli_oracle.c.
"""
