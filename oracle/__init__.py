"""CPU oracle for one Medusa draft-and-verify step.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, float64 NumPy
statement of what one verify step computes. Only the test suite, the smoke
check of ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it. The HIP library and its Python binding never import, call or link
anything here, and nothing here imports them.

Sources (web pages, cited by title and section):

* "Medusa: Faster LLM text generation" (nazmi.tech) -- Inference, Tree
  attention, Acceptance rules.
* "Medusa 深读：解码慢不是算力问题，是搬运问题" (jokeuncle.pages.dev) -- §3.1
  head equation, §3.2 independence, §5 typical-acceptance equation and rule
  table, §6.1 tree and node-count equation, §6.2 sparse tree and its worked
  example.
* "Medusa Part I: Architecture, Training, and Shifted Loss"
  (sudhirpol522.github.io) -- Part 2 (greedy verification, progress
  guarantee), Part 3 (ResidualBlock / MedusaHead).

Modules:

* ``numerics``   -- bf16 storage semantics (exact widening, rounding points)
* ``heads``      -- Medusa heads, top-s pools, head log-sum-exp
* ``tree``       -- candidate tree: node count, topology, mask, retrieve, tokens
* ``verifier``   -- one-layer synthetic verifier, tree attention (two ways), LM head
* ``posterior``  -- greedy / typical / exact acceptance, longest prefix, commit
* ``step``       -- the whole step composed from the above
* ``sparse_tree``-- calibrated sparse-tree greedy builder (a next-step row)

Parity status: the verifier internals (embedding, QKV, RoPE, O-projection,
LM head of the synthetic layer) are not defined by the pages; they are parity
unpinned beyond the tree-attention path-equivalence invariant.
"""

from . import numerics, heads, tree, verifier, posterior, step, sparse_tree  # noqa: F401
