"""CPU oracle for ragged paged attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct reference implementations in float64 (numpy)
and pure Python.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package;
the product path (``decode_attention_kv_pd_amd``) never does, and this package
imports nothing from it.

Modules
  attention  float64 softmax attention over logical (unpaged) K/V
  brute      the same definition in pure-Python scalar loops (tiny inputs)
  paged_kv   page-level append / gather / pack / unpack on a numpy pool

What each function follows is cited in its docstring: the Perplexity post
"Disaggregated prefill and decode" (sections "Prefill vs Decode
performance", "KV Messenger", "Sharded KV Cache Transfers", "Speculative
Decoding", "Qwen3-Coder") and the kwkr.cn PD-disaggregation survey
(sections 5.1 and 8).  The pages never write the attention formula out; the
oracle uses standard scaled-dot-product softmax attention, with the causal
mask aligned to the end of the cache (query i of a request with qo new tokens
over kv cached tokens sits at absolute position kv - qo + i).

Every function here is pinned by the CPU tests in ``tests/test_oracle_*.py``
(brute force, closed forms, invariants, a library routine, the survey's
transfer-size example, and planted mutants that the pins must catch).
"""

from . import attention, brute, paged_kv  # noqa: F401
