"""CPU fp64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
anything in this package; only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library.

Sources (pages are cited by title and section):

* [CANN-FA] "FlashAttention in CANN ops-transformer on the Ascend NPU"
  (hwcomputing.csdn.net): the standard-attention formula and code in the
  section on where the memory black hole comes from; the softmax definition
  and the blockwise online-softmax pseudocode in the section on online softmax;
  the mask modes in the tuning section.
* [YOLO11-FA2] the lpnh.cn article on swapping YOLO11's attention for a
  FlashAttention-2 style kernel: section 2.2 (online softmax is exact),
  section 2.3 (backward recomputes S and P), section 3.2 (Q-block loop).
* [FA-GQA] "Transformer高效注意力机制实现：Flash Attention与GQA原理对比与代码实践"
  (yunthe.com): the MHA class and the GQA class (repeat_interleave of K, V);
  its KV-cache discussion motivates the decode reference (``ref_decode``).

* Philox-4xW-R: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
  easy as 1, 2, 3" (SC'11), the counter-based generator both the kernels and
  ``philox.dropout_keep`` implement for the fused dropout that [CANN-FA]'s
  tuning section recommends.

Every function here is pinned by CPU tests in ``tests/test_oracle_*.py``
(brute force, hand-worked closed forms, invariants, finite differences).
"""

from .attention import (  # noqa: F401
    ref_fwd,
    ref_bwd,
    ref_fwd_head,
    ref_bwd_group,
    blockwise_online_fwd,
    kv_head_of,
    allowed_mask,
    ref_decode,
)
from . import philox  # noqa: F401
