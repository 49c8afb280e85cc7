"""CPU oracle for the Recurrent Looped Transformer forward pass.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.
"""
from .rlt_oracle import Oracle, OracleState, log_softmax64, V0, V1, V2  # noqa: F401
