"""CPU oracle for AB-Attention's block-sparse attention path.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the library under
``block_sparse_attention_ibcs_amd`` never does, and it shares no code with it.

What it computes follows the AB-Attention abstract (paperdot search page,
query "Xing Ma"): dynamic block-sparse attention that computes exact attention
only on key/value blocks chosen from the current activations (problem
sentence), scored by clustering the queries of each query block in place,
token order untouched (IBCS sentence), drawn with probabilities proportional
to those scores and
given weight 1/pi (pi the block's inclusion probability), which makes one
weighted pass an unbiased estimate of the dense numerator and denominator
(SIP sentence). The pages give no formulas; every constant and rule
the abstract leaves open is a stated reading, listed in the module that uses it.

The INTRA relay patterns (``intra``) follow the INTRA page (paperdot search page,
query "Wenbo Lu"): static Scatter / Gather kept lists under a partition model,
an alternative index producer for the same weighted attention.

The FP8 variant (``fp8``) follows the VC-Attention page (iitak.ru news on
MiniMax-H3): 8-bit products, V-Smooth (per-block mean subtracted, residual
quantised) and ExpCast-FP8 (the FP8 byte of a probability from one linear
formula with rounding); quantisation codes are exact, the attention is float64.

Precision: k-means is an exact-operation fp32 specification (both sides must
produce identical bits), the sampler is integer arithmetic on fp32 scores, and
everything else is float64.

Pins (what fixes each function against something other than itself) live in
``tests/test_oracle_*.py``. No function here is "parity unpinned".
"""

from .philox import philox4x32_10
from .ibcs import kmeans_fp32, block_scores, round_bf16
from .sip import quantize_scores, budget, inclusion_thresholds, sample_rows, SIP_ONE
from .topk import topk_rows
from .systematic import sample_rows_systematic
from .attention import dense_attention, sparse_ht_attention
from .pipeline import Params, run_blocks
from . import fp8
from . import intra

__all__ = [
    "philox4x32_10",
    "kmeans_fp32",
    "block_scores",
    "round_bf16",
    "quantize_scores",
    "budget",
    "inclusion_thresholds",
    "sample_rows",
    "topk_rows",
    "sample_rows_systematic",
    "SIP_ONE",
    "dense_attention",
    "sparse_ht_attention",
    "Params",
    "run_blocks",
]
