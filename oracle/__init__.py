"""CPU float64 oracle for SANTA++ sampled-team decode attention.

TEST INFRASTRUCTURE. This package is the slow, plain reference that the HIP
path is checked against. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does, and
it imports nothing from the product package.

Sources it follows (cited by title and section in every function):
  [ABS]  "SANTA++: Sampling Attention through Representative Keys",
         arXiv 2609.35629, abstract (arxivdaily.com and fugumt.com pages).
  [EXP]  "SANTA++：用代表性 Key 采样把 KV cache 读带宽砍掉 80%" (explainer page,
         papers.ananclaw.com), section 三 "核心方法" and its sub-sections.
  [PHX]  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
         1, 2, 3", SC'11, the Philox generator family (Philox4x32, 10 rounds).

Every function states which of these it follows. Where a source leaves a step
open the reading taken is stated in the function's docstring.

Parity status of each function (what pins it) is listed in the header of
``santa.py``.
"""
from .philox import philox4x32_10, draw_words, word_to_uniform  # noqa: F401
from .numerics import decode_bf16, round_to_bf16, round_to_dtype  # noqa: F401
from . import santa  # noqa: F401
