"""CPU oracle for DeepSeek-V4's hybrid compressed attention (CSA + HCA).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.  The
HIP library and its Python binding never import it, and it imports nothing from
them: the two share no code.

The oracle is a plain, slow, direct evaluation of the definitions in fp64
(numpy), starting from the same stored bytes the kernels read.  Every function
cites the page passage it follows; the pages print no formula, so each formula is
a reading, and the readings are listed in the repository's design notes.

Pages cited (by title, with their site):
  * "DeepSeek V4 infrastructure" (volanea.com), section "Compression only works if
    the attention path is engineered end to end";
  * "DeepSeek Releases V4 with Million-Token Context Optimized for AI Agents"
    (botbeat.news), section "Summary";
  * "Inside DeepSeek V4: How a Resource-Constrained Team Engineered a Million-Token
    AI Giant" (jakobijn.be), section "The Architecture: Hybrid Attention (CSA + HCA)";
  * "DeepSeek V4: How They Crushed the Million-Token Memory Problem"
    (sameershanbhag.com), section "Two kinds of memory instead of one".
"""
from . import quant, rope, pool, indexer, topk, attend, step, prologue, project  # noqa: F401
