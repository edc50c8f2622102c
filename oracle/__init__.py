"""Plain CPU oracle for the DeepSeek Sparse Attention (DSA) hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, headers, tables or helpers with the
HIP library in ``sparse_long_context_dsa_amd/``; the two meet only through the
seeded input generator in ``workloads/``, which holds none of the method's
arithmetic.

Everything is NumPy in float64 after an exact decode of the FP8 / bf16 inputs.
The method reaches a plain definition exactly (no approximation), so each
function is that definition written out:

* ``fp8``      - OCP FP8 E4M3 ("fn") codec and the per-row absmax/448 quantiser.
* ``bf16``     - exact bf16 decode.
* ``layout``   - logical position -> physical cache row (contiguous or paged).
* ``dsa``      - lightning-indexer scores, top-k selection, sparse and dense
                 MQA-mode MLA attention, and their composition.
* ``kl``       - the indexer's training loss: the head-summed attention target,
                 KL(target || Softmax(I)) and the gradients with respect to the
                 indexer's scores and inputs.

Sources are the web pages on DeepSeek Sparse Attention; each function names the
page and the section or equation it follows.
"""

from . import bf16, dsa, fp8, kl, layout  # noqa: F401
from .bf16 import bf16_decode  # noqa: F401
from .dsa import (  # noqa: F401
    dense_mla,
    forward_query,
    indexer_scores,
    indexer_scores_query,
    sparse_mla,
    topk,
)
from .fp8 import E4M3_MAX, e4m3_decode, e4m3_encode, e8m0_decode, quantize_rows, quantize_rows_e8m0  # noqa: F401
from .kl import (  # noqa: F401
    attention_target,
    dequantise,
    indexer_backward_query,
    indexer_kl_query,
    indexer_logits,
    kl_to_softmax,
)
from .layout import phys_rows  # noqa: F401
