"""CPU oracle for exact softmax attention (forward and gradients) -- TEST
INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in the package entry file and the
``cpu_baseline`` leg of the bench script may import anything in this
package.  The product path (the HIP library and its Python binding) never
calls it, and this package never imports the product path: the two share no
code.  Inputs reach both sides from the seeded generator module, which holds
none of the attention arithmetic.

Contents
--------
``attention``  NumPy float64 implementation of the plain definition, in row
               blocks restricted to each block's visible key span.
``brute``      Pure-Python double loops with ``math.fsum``, tiny shapes only;
               it pins ``attention``.
``backward``   NumPy float64 gradients (dQ, dK, dV) of the same definition,
               by the chain rule; pinned by central finite differences of the
               forward oracle, by float64 autograd through masked SDPA and by
               closed forms.
``general``    NumPy float64 attention over packed variable-length sequences
               with causal / window / band / global-token masks; pinned by the
               forward oracle per sequence, by a per-pair brute force and by
               closed forms.
``fp8``        OCP E4M3 rounding, byte codes and power-of-two per-tensor
               scales, and the exact attention of the dequantised tensors;
               pinned by the format's closed-form values, a brute-force
               nearest search with ties to even, and torch's float8_e4m3fn.
``decode``     NumPy float64 decode attention over a paged KV cache (gather
               through the page table, then the plain definition), and the
               rule that merges results over disjoint key sets; pinned by the
               forward oracle on the equivalent contiguous cache, by the
               brute force and by page-permutation and sharing invariants.

What the oracle computes (the plain definition; every page agrees that the
tiled method returns exactly this result):

* "Efficient attention: long context and sub-quadratic variants", section
  "What it is and when you reach for it": out = softmax(QK^T / sqrt(d)) V.
* "Efficient Attention: FlashAttention, Sparse, Linear", section 45.2.1
  (the displayed Attention(Q, K, V) equation).
* Same first page, section "Implementation, twice": masked entries are set
  to -inf before the softmax, so they get exactly zero weight and each row
  renormalises over its visible set; the sliding window lets row i see keys
  j with i - w < j <= i.
* "Attention Mechanism Variants Beyond Self-Attention", section
  "Multi-Query and Grouped-Query Attention": KV heads are repeated with
  ``repeat_interleave`` so query head h reads KV head h // (Hq / Hkv).

The per-row logsumexp is not defined on any page.  Reading used here: the
natural-log logsumexp of the *scaled* scores over the row's visible set, so
that p_ij = exp(s_ij - lse_i).  It is pinned by closed forms (uniform
weights give ln|V_i|; one-hot retrieval gives ln(e^a + n - 1)) and by
``torch.logsumexp`` over explicitly masked float64 scores.

Every function here is pinned by tests that do not re-type its formula; no
function in this package is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_forward,
    attention_rows,
    kv_head_of,
    visible_span,
)
from .backward import attention_backward  # noqa: F401
from .decode import decode_paged, gather_pages, merge_partials  # noqa: F401
from .general import attention_general, visible  # noqa: F401
from . import fp8  # noqa: F401
from .brute import brute_attention  # noqa: F401
