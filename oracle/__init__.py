"""CPU oracle for the CSA / HCA attention path — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct float64 NumPy statement of what the
library computes.  It is imported only by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``;
the product path (the HIP library and its Python binding) never imports,
calls or falls back to anything here, and this package shares no code,
tables or helpers with it.

Sources followed (the pages describe the method in prose only, without
formulas; every constant that the prose leaves open is a stated reading):

* honbul.tistory.com/221 ("DeepSeek-V4: Towards Highly Efficient Million-Token
  Context Intelligence 논문 정리"), sections "CSA: 압축한 뒤, 필요한 기억만 골라서
  보기", "HCA: 더 강하게 압축하고, 압축된 전체를 보기" and "KV cache를 줄이는
  방식: 저장 구조까지 바꾼다".
* pogovet.com ("DeepSeek-V4: a million-token context that agents can actually
  use"), 상세 정리 §4 "CSA와 HCA를 결합한 하이브리드 어텐션" and §5 "층 배치와
  저정밀 저장이 만드는 누적 효과".

Modules:
  codecs  – exact decoders/encoders for bf16, OCP fp8 e4m3 and OCP MXFP4.
  method  – compression, indexer scores, top-k, CSA/HCA attention, LSE merge.
  brute   – a dense-mask, loop-based restatement for tiny inputs (a pin).

Every function is pinned by ``tests/test_oracle_pins.py`` (closed forms,
invariants, worked examples with literal numbers, library routines).
"""
from . import codecs, method, brute  # noqa: F401
