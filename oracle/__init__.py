"""CPU float64 oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  It shares no code with the HIP library
and imports nothing from it.

Pages cited throughout (by title and section):
  [FA-legal]  inferensys.com glossary "FlashAttention" (legal pre-training):
              paragraphs on IO-awareness, online softmax, backward
              recomputation, FlashAttention-2/-3, memory scaling; glossary
              entries "IO-aware", "Online softmax", "Memory hierarchy",
              "Recomputation", "Block-sparse".
  [Digest]    "Paper digest: FlashAttention": "Why this paper exists",
              "Method, without the wall of equations", "Limits".
  [IO-aware]  chipfoundryservices.com "flash attention io aware": "The Memory
              Bandwidth Bottleneck", "Flash Attention Algorithm", "Online
              Softmax", "Performance Impact" table, "Integration".
  [FA-LLM]    inferensys.com glossary "Flash Attention" (self-hosted LLMs):
              opening paragraphs; entries "Grouped-Query Attention (GQA)",
              "KV Cache" and "PagedAttention".

Dropout (``dropout.py``) also follows a published definition outside the
pages: the Philox4x32-10 counter-based generator of Salmon et al. (SC 2011),
pinned to that generator's published known-answer vectors.

Parity pins: every function here is pinned by a ``-m "not gpu"`` test against
closed forms, invariants, finite differences, a library routine (torch CPU
float64 scaled_dot_product_attention) or the pages' printed memory arithmetic.
No function is "parity unpinned".
"""
from .attention import (  # noqa: F401
    BlockMask,
    forward,
    forward_online,
    decode_forward,
    decode_paged_forward,
    backward,
    probabilities,
    head_rows_forward,
    head_rows_backward_dq,
    head_full_stats,
    head_cols_backward_dkdv,
    attention_matrix_bytes,
)
from .fp8 import e4m3_decode, e4m3_encode_rne_sat, quantize_per_tensor, E4M3_MAX  # noqa: F401
from .dropout import (  # noqa: F401,E402
    backward_dropout,
    drop_probability,
    drop_threshold,
    forward_dropout,
    head_backward_dropout,
    keep_mask,
    philox4x32_10,
)
