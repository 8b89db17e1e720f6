"""CPU oracle for the MX-quantised MoE expert block — TEST INFRASTRUCTURE.

A plain, slow, obviously correct fp64 implementation of what the GPU path computes: MX codecs
(`oracle.mx`) and the block itself, step by step (`oracle.moe`). It exists to check the GPU path
and nothing else: only tests/, the package's smoke check and the bench's CPU-baseline leg may import
it. The GPU path never imports, links or calls anything here, and nothing here imports the GPU
path; the two share only the seeded input draws of the `workloads` module.

Pins (tests/test_oracle_*.py, run on the CPU) tie every function to something other than itself:
hand-computed MX blocks and library fp8 casts for the codecs, brute force and closed forms for
routing and the sort, a dense all-expert evaluation, a dense-MLP shared-expert identity,
permutation invariance and textbook special cases for the whole block.
"""
from . import mx, moe  # noqa: F401
from .moe import (route, align, align_capacity, moe_block, ExpertWeights, Layout,  # noqa: F401
                  parity_stats)
