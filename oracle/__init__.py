"""fp64 CPU oracle for the MoE FFN-service layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP path.

Parity status of each function is stated in ``afd_oracle``'s header.
"""
from .afd_oracle import *  # noqa: F401,F403
