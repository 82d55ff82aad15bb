"""CPU oracle for token-tree verification -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct implementation of what the verification
path computes, in float64 for floating point and exact integers elsewhere.
Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the product path never does, and it shares no code
with the GPU kernels (it imports neither the package nor its sources).

Pages it follows (cited by title and section in each function):

* "Beam Search、约束解码与 Tree/Self Speculation" (decoding-extensions glossary,
  llm-glossary.tokens-kit.com): sections "Tree/Self Speculation", "Packed tree
  attention", the packed-vs-branch experiment and the three-part semantics
  experiment (verify_tree).
* "投机解码的树状注意力验证" (tree-attention verification essay, wiblog.cn):
  sections on the custom attention mask and on KV cache / batching.
* "02 · Token Tree 与 Tree Attention" (llm-infra-atlas): section 2 (token tree
  definition), 3 (mask rules, positions example), 4 (verify flow).
* "Accelerating Speculative Decoding with Block Diffusion Draft Trees" (DDTree
  notes): sections 4-5 (top-B prefixes, Lemma 1, the best-first heap), 6
  (worked example) and 7 (tree attention, verifier walk, temperature
  sampling, losslessness).
* "解码：采样、束搜索和推测性解码" (decoding page): section "Gumbel Max技巧".

Modules: ``bf16`` (bit-level bf16 <-> float64), ``tree`` (metadata),
``attention`` (per-node linearised-path causal attention), ``accept``
(argmax + sequential greedy walk), ``commit`` (copy-based commit/rollback),
``sampling`` (temperature-sampling walk by Gumbel-max; stochastic
min(1, p/q) walk), ``ddtree`` (DDTree's best-first top-B draft tree).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against values the pages print, closed forms or brute force; the exact
numeric attention values on the synthetic workloads are checked only against
this float64 definition (there is nothing else printed to pin them to).
"""

from . import bf16, tree, attention, accept, commit, sampling, ddtree  # noqa: F401
