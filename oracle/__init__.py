"""CPU oracle of the MXFP4 routed-expert MoE layer: plain C++17 in fp64
(moe_oracle.cpp, moe_oracle.h; the command-line tool moe_oracle_cli.cpp),
with thin Python wrappers.

TEST INFRASTRUCTURE: a plain, slow, obviously correct implementation that the
HIP path is checked against.  Only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may import it; the product path never does, and
this package never imports the product package.

  oracle.mxfp4  number formats (E2M1/E8M0 decode and quantise, bf16 rounding)
  oracle.mxfp8  E4M3 elements (MXFP8 weights)
  oracle.moe    route, align, router GEMM, expert MLP, forward
  oracle._lib   builds (g++) and loads the C++ library
"""
from . import mxfp4, mxfp8, moe  # noqa: F401
