"""Oracle for the paged-KV attention and relayout path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
CPU model of what the GPU path computes.  Only the test suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  The product path (``decode_paged_kv_amd``) never imports,
calls or links anything here, and this package imports nothing from it: the
two share no code.  Inputs reach the oracle as plain numpy arrays.

Pages cited in this package (titles as they appear on the pages):

* [MUX]    "PD multiplexing: splitting prefill and decode by SM on one GPU"
           (AI-infra handbook, serving / frontier chapter; English and
           Chinese editions carry the same content).
* [DISAGG] "PD 分离与 KV 传输" (PD disaggregation and KV transfer,
           AI-infra handbook, serving / distributed chapter).
* [L7]     "Lecture 7 · Prefill 与 Decode：分块 prefill、解耦与 NVIDIA
           Dynamo" (CS349D lecture-7 notes).
* [EPD]    "推理 INFRA 方法论（6）：PD 与 EPD".

Modules:

* ``attention`` - exact causal GQA softmax attention in float64 (prefill
  rows and decode rows are the same function of absolute position).
* ``pool``      - a host model of the paged KV pool: slot mapping, the naive
  per-token write, gather, and the naive per-(token, head) relayout.
* ``policy``    - the PD-multiplexing split / level / layers-per-round rules.
* ``accounting``- closed forms: KV bytes, chunked-prefill KV re-reads, the
  causal attention flop count and the decode byte count.
"""

from . import accounting, attention, policy, pool  # noqa: F401
