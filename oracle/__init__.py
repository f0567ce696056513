"""CPU oracle for low-bit (SageAttention-style) quantized attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants
module, table or helper with the HIP library under
``bit_quantized_attention_sage_amd/``; the two meet only through the seeded
inputs that ``workloads.py`` produces.

What the pages fix, and what they leave open
--------------------------------------------
The pages ("Faster! Even faster! ..." podcast notes, section "02:48 There were
clearly faster compute units on the hardware"; the Vidu S1 technical blog,
section "Infra") say only that SageAttention is low-bit quantized attention
that replaces FlashAttention as a drop-in ("37:54 One line of code, twice the
speed"), and that streaming generation attends causally frame by frame to a
KV cache (blog, sections "模型架构" and "训练方法").  They give no bit width,
block size, smoothing or rounding rule.  The oracle therefore has two levels:

* ``attention.attention_fp64`` -- the plain definition of the result being
  approximated: softmax(Q K^T * scale + mask) V in float64.
* ``quant`` + ``emulate`` -- the quantization scheme this library states as
  its own design (INT8 Q/K with K mean-smoothing and per-block scales; P.V in
  the input's 16-bit type or in FP8 e4m3 with per-32-key E8M0 V scales),
  written out step by step on the CPU.

Every function below cites the passage, or the stated reading of it, that it
follows.  Parity of the quantized path against the pages themselves is
unpinned: the pages print no operator-level value or worked example.
"""

from . import codecs, fp32, quant, attention, emulate  # noqa: F401
from .constants import *  # noqa: F401,F403
