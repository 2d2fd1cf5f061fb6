"""CPU oracle for mixed-head (retrieval / streaming) attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link or
execute anything in this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP library
(``mixed_head_kv_amd``); the only thing both sides consume is the seeded input
generator module ``mixed_head_kv_amd.inputs``, which holds no attention arithmetic.

Contents
--------
``attention``  fp64 masked-softmax attention over the full K/V history, with the
               retrieval / streaming visibility rule (plain definition).
``int4``       the group-128 asymmetric int4 KV codec with fp16 scale and zero
               (plain definition, fp32 steps as the format fixes them).
``linear``     the 8-bit-weight linear layers around the attention (fused QKV
               projection with the rotary encoding, output projection), fp64.

Every function cites the passage of the source pages it follows.  The pages are:

* "DuoAttention: Efficient Long-Context LLM Inference with Retrieval and Streaming
  Heads" (hotpaper.ai summary page): the abstract, and the Korean sections
  on the technical approach and the main results.
* "What is DuoAttention" (nav.superapi.store): "Technical principles of DuoAttention".
* "韩松团队长上下文LLM推理高效框架:单GPU 330万Token上下文推理" (cn.bg3.co): the sections
  on the research background and on DuoAttention's design.
* "DuoAttention是什么？" (zhuoshang.net): "DuoAttention的技术原理".
* the AIxiv column repost on takechan.xyz (garbled copy of the cn.bg3.co article).

Pins: every function here is checked by ``tests/test_oracle_*.py`` against library
routines, closed forms, brute force and invariants (none of them re-typing the
oracle's own formula); no function is "parity unpinned".
"""

from . import attention, int4, linear  # noqa: F401
