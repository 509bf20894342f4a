"""CPU oracle for the Medusa verify step -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy code (fp64 unless stated) that defines
what the HIP path must compute.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code
with the HIP library (``medusa_tree_verification_amd``) and imports nothing
from it; the two meet only through the seeded input generator.

Pages cited (each function names the page and the section it follows):

  P1  "Medusa 심층 아키텍처: 별도 초안 모델을 제거한 다중 헤드(Multi-Head) 추측
      디코딩과 Tree Attention 3배 가속 원리" (techknowgenie.com)
  P2  "[vLLM] Medusa: 다중 예측 헤드 투기적 디코딩" (blog.secrett2633.cloud)
  P3  "Speculative Decoding(투기적 디코딩) 원리와 가속 아키텍처: Draft Model과
      Rejection Sampling부터 Medusa·EAGLE-3 및 vLLM 서빙 최적화까지" (blog.huny.dev)
  P4  "최적화 2편. 추측 디코딩과 긴 컨텍스트 - Speculative Decoding과 MEDUSA·EAGLE,
      Ring Attention" (beengineer500.github.io)

Modules:
  heads      residual SiLU block + vocab projection            (P1, heads)
  topk       per-head top-k                                    (P1, sketch code; P2, propose())
  tree       static tree, ancestor sets, mask, tree tokens,    (P1, tree attention; sketch code;
             expected accepted length, optimal tree (brute)     P2 paper results)
  attention  tree-masked attention, path-causal alternative    (P1, tree attention; P4 3.3)
  accept     greedy and rejection-sampling acceptance          (P1, rejection sampling; P3 2, 5; P4 1.3)
  step       the four stages composed
  commit     KV rollback / compaction after acceptance; greedy decoding (P3 5; P4 1.3)
  dense_heads  the heads on every tree row (M = B*T) and each head's top-k (P1, heads; sketch code)

Every function has at least one pin in ``tests/test_oracle_*.py`` that ties it
to something other than itself (worked examples printed on the pages, closed
forms, brute force, alternative definitions, library routines).
"""
from . import heads, topk, tree, attention, accept, step  # noqa: F401
