"""Plain CPU oracle for one EAGLE-style draft-tree round (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only the tests, the smoke check of the graft entry point and
the CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
path; the only module both sides import is the seeded input generator `synth`,
which holds no arithmetic of the method.

Each function follows the passage of the pages that defines it:

* "EAGLE: Speculative Sampling Requires Rethinking Feature Uncertainty"
  (papercache.org notes): background section A3 (the speculative-sampling
  acceptance rule min(1, p/q), resampling from norm(max(0, p - q))), section
  3.3 (tree verification, recursive speculative sampling at every node),
  appendix A.1 (greedy: top-k children; non-greedy: k sampled children) and
  appendix A.2 (multi-round speculative sampling over k candidates).
* "EAGLE-2: Faster Inference of Language Models with Dynamic Draft Trees"
  (tom-jerr.github.io notes): "Expanding the Draft Tree" (value equation
  V_i = prod confidence, top-k frontier of the current layer), "Rerank draft
  tokens" (top-m by value, shallower wins ties, connected result),
  "Tree Attention Mask" (flatten, ancestor-only visibility).
* "LLM 推测性解码原理解读" (hubwiz.com): section 1 (accept/correct rule, bonus
  token, at least one and at most draft+1 committed tokens), section 2 (output
  distribution unchanged; temperature adjusts both distributions) and section 5
  (one verify pass scores every root-to-leaf path as if independent).

Readings of points the pages leave open are listed in the design notes; the
ones each function relies on are restated in its docstring.
"""

