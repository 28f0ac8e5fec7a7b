"""CPU oracle of the MXFP4 routed-expert MoE layer (numpy, fp64).

TEST INFRASTRUCTURE: a plain, slow, obviously correct implementation that the
HIP path is checked against.  Only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may import it; the product path never does, and
this package never imports the product package.

  oracle.mxfp4  number formats (E2M1/E8M0 decode and quantise, bf16 rounding)
  oracle.moe    route, align, expert MLP, combine, forward
"""
from . import mxfp4, moe  # noqa: F401
