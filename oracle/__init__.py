"""Plain CPU oracle for the paged KV-cache hot path (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing in the product may import this package:
only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` call it.  It shares no code with the HIP library or its Python
binding; every function is written out from the definitions on the pages it
cites, slowly and plainly, so that a reader can check it against them by eye.

Sources (web pages; cited by title and section):

* "Deep Dive into vLLM Worker-Side GPU KV Cache Initialization"
  (kongchang.com, English) -- called *Worker-Side KV Init* below.
* "vLLM의 KV cache 연결 흐름" (llm-engineer.pages.dev card
  vllm-kv-cache-engine-to-worker, Korean) -- *Engine-to-Worker card*.
* "Understanding PageAttention Memory Optimization" (freaks.city blog,
  English) -- *PageAttention blog*.
* "vLLM Worker侧GPU KV Cache初始化流程深度解析" (kongchang.com, Chinese
  original of the first page, with extra paragraphs) -- *Worker-Side KV Init
  (zh)*.

Modules:

* :mod:`oracle.paging`    -- slot mapping, cache write, gather by block table.
* :mod:`oracle.e4m3`      -- the OCP FP8 E4M3 ("FN") codec.
* :mod:`oracle.int4`      -- the 4-bit integer codec (zero point 8, packed).
* :mod:`oracle.bf16`      -- bf16 <-> float conversions from the bit layout.
* :mod:`oracle.attention` -- softmax attention over a paged cache (fp64).
* :mod:`oracle.sizing`    -- KV bytes-per-token and pool-size closed forms.
* :mod:`oracle.layout`    -- hybrid KV groups / shared tensors / SWA release.

Pin status: every function here is pinned by a ``-m "not gpu"`` test against
values the pages print, closed forms, library special cases or brute force.
No function is "parity unpinned".
"""

from . import bf16, e4m3, int4, paging, attention, sizing, layout  # noqa: F401
