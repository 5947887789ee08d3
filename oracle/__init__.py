"""CPU oracle for one Medusa decode step — TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 numpy code that computes what the method computes, step by
step, so that the GPU library can be checked against it.  Only the tests, the
smoke check and the CPU-baseline leg of the benchmark may import it; the GPU
library never calls it and shares no code with it.

Sources (the web pages on Medusa this work is built from):

* Ultralytics glossary, "Medusa Heads" — section "Comment les têtes prédisent
  les tokens suivants" (head formula, zero-init example) and section
  "Attention arborescente et acceptation" (Cartesian candidate tree, ancestor
  mask, greedy acceptance, longest accepted branch, sparse 64-node tree).
* aiunderstanding.org, "Medusa Decoding Heads" — section "Diepe duik"
  (lossless: accepted text equals what greedy decoding would produce).
* codewithpapers, "Medusa: Simple LLM Inference Acceleration Framework with
  Multiple Decoding Heads" — abstract (tree-based attention verifies all
  candidates in one step).
* testnode25 blog, "Medusa no contexto de LLMs" — section "o que significa
  medusa na prática de deploy" (fall back to the conventionally generated
  token when a candidate is rejected).

Every function below is pinned by a CPU test against something other than
itself (closed forms, brute force, a library routine on a special case, or the
page's printed output); see each function's docstring for its pin.
"""
from .medusa_ref import *  # noqa: F401,F403
from .plan_ref import *    # noqa: F401,F403
