"""CPU oracle for the TQ4_1S / NVFP4 / MXFP6 weight path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: it is used by ``tests/``, by
``__graft_entry__.smoke()`` (to check one GPU result) and by the
``cpu_baseline`` leg of ``bench.py``.  It shares no code, header, table or
constant generator with the HIP library; the two meet only through the seeded
input generators in ``workloads.py`` and through the arrays a test hands to
both.

Implementation rules followed throughout:

* plain numpy (plus the Python standard library); float64 for the
  mathematics, and a *canonical float32* quantizer whose operation order is
  fixed so that a GPU implementation can be compared with it bit for bit
  (numpy's float32 ``+ - * /`` and ``sqrt`` are IEEE-754 correctly rounded and
  are never contracted into FMAs);
* no blocking, fusion or reordering beyond what the definition states.

Sources cited in the docstrings (the text of five web pages):

* **TQ4 page** -- the page at hotelren.com/news/5458160, whose (unrelated)
  title is "企业官网建设流程全解析"; its body summarises community results for
  TQ4_1S weight compression in a llama.cpp fork.  Sections used:
  "TQ4_1S 是什么" (what TQ4_1S is) with its sub-list "格式原理" (format
  principle, items 1-3 and the paragraph after them); "解码速度：分硬件汇总"
  (decode speed by hardware) with the paragraph on why CUDA differs; and
  "适用前提与边界" (preconditions and boundaries).
* **Quantizer-tool page** -- bittide.aicompass.dev, titled "这是我的 llama.cpp
  NVFP4/MXFP6 GGUF 量化工具" (an NVFP4/MXFP6 GGUF quantizer); sections
  "目前能实现的部分功能" (features), "RSF" and "MXFP6 的未来" (MXFP6's future).
* **llm-compressor page** -- ai-insight.org/news/11771, which names NVFP4 as
  NVIDIA's 4-bit float format introduced with Blackwell (section
  "NVFP4 + FP8 双格式支持").

The pages define the *structure* of TQ4_1S (32-element blocks, a randomized
Hadamard rotation with sign flips, a 16-level Lloyd-Max codebook for N(0,1),
4-bit indices, two half-block scales d0/d1, no correction term) but print no
bit layout, sign vector, scale statistic or rounding rule, and NVFP4/MXFP6 are
only named.  Every reading taken where the pages are silent is stated at the
function that takes it.

Parity status per function (what pins it is in ``tests/test_oracle_*.py``):
all functions exported here are pinned; nothing is "parity unpinned" except
bit-compatibility with the llama.cpp fork's own files, which this package
does not claim.
"""

from . import codebook, tq4_1s, minifloat, blockfp, q8, rsf, kv  # noqa: F401
