"""CPU oracle for the LampAttention forward pass -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct NumPy model of what the
look-ahead mixed-precision FlashAttention forward pass computes, written from
"LampAttention: Look-Ahead Mixed-Precision FlashAttention for Dedicated
Accelerators" (abstract; tables 1-6 "16-bit sub-blocks per tile"; figures 1-8
captions for the delta / tau parameters).  It exists so that the HIP path can
be checked against it.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in here.  The product path (the C-ABI
library and its Python binding) never does, and this package imports nothing
from the product path: the two share no code.  Inputs reach both sides from the
separate seeded generator module ``inputs``.

Modules
-------
formats  software e4m3fn / bf16 / fp32 rounding on exact fp64 values
lamp     the tiled LampAttention forward pass, step by step
refs     endpoint references: exact fp64 attention, plain bf16 attention
brute    scalar brute force of the whole method for tiny inputs, written
         independently of ``lamp`` (exact rationals for every rounding)

Parity status: every function is pinned by a ``-m "not gpu"`` test
(tests/test_oracle_*.py).  The 16-bit logit ``acc16`` is an fp64 dot product
rounded to fp32; it equals the correctly rounded exact sum except when the
fp64 sum lies within fp64 error of an fp32 rounding boundary (documented, not
a parity hole: outputs are compared with a tolerance).
"""
