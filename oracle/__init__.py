"""fp64 CPU oracle for exact tiled attention.

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and bench.py's
``cpu_baseline`` leg may import, call or execute anything in this package.  It
is independent of the HIP library: no code, headers, tables or constants are
shared between the two; the only common input is the seeded generator module
``tiled_exact_attention_bf16_amd.inputs``, which holds no attention arithmetic.

Modules:
  attention       plain-definition forward (O, LSE) and backward (dQ, dK, dV)
  online_softmax  tiled streaming model with the lazy rescaling threshold
  exp2_split      model of the FMA-only exp2 (integer/fraction split + cubic)
  schedule        longest-first ordering of query tiles by the keys they visit
"""
from . import attention, online_softmax, exp2_split, schedule  # noqa: F401
