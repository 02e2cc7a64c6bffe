"""CPU oracle for the tree-verification pass with W12 weights.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

What it computes is written out from the pages' description of the method
(page "SpecPilot이 배포 환경마다 추측 디코딩 병목을 스스로 찾아 10.87배까지
끌어올린다", onedev.kr, abbreviated below as *SpecPilot summary*):

* ``w12``     -- the lossless 12-bit weight format (SpecPilot summary,
                 section 무엇과 다른가 / "how it differs");
* ``model``   -- plain greedy inference of a dense decoder with bf16 weights,
                 one pass over every draft-tree node (section 무엇인가 /
                 "what it is": the target checks the drafter's tokens in one
                 forward pass), plus the definition-level per-path variant;
* ``accept``  -- the matched path and bonus token (section 무엇과 다른가);
* ``lmhead_i8`` -- the LM head on INT8 weights with a Cauchy-Schwarz
                 certified candidate filter, exact argmax kept (section
                 무엇과 다른가);
* ``gdn``     -- Gated DeltaNet layers of a hybrid target over a draft tree:
                 every node's output with the state recomputed along its
                 root path, and the state after the accepted path (section
                 무엇과 다른가);
* ``tlv``     -- two-level verification: a Q pass on the 8-bit leading view
                 of the W12 records, then one exact pass over the matched
                 path, the bonus token and a re-drafted subtree (section
                 무엇과 다른가).

Floating point is fp64 between the bf16 rounding points the method fixes
(bf16 inputs and outputs of every op), so the oracle is at least as accurate
as any fp32-accumulating kernel it is compared with.

Parity pins are in ``tests/test_oracle_*.py``.  Absolute logit values of a
random-weight model have no worked example on the pages: their only pins are
the structural ones listed there (library-routine equivalences, closed forms,
special cases), which is stated where it matters.
"""

from . import bf16, w12, accept, model, tlv, lmhead_i8, gdn  # noqa: F401
