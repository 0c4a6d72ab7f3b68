"""The oracle's decoding loop on planted agreement: what the loop must do is
fixed by the construction, independently of the oracle's stages. With a
permutation language pi (the verifier's next token after t is pi(t)) and
each head's true continuation planted at a known rank, every step must
commit the chain root, pi(root), pi^2(root), ... of exactly the length the
tree allows — the deepest tree path whose ranks are the planted ranks of the
token the step starts from — and hand pi of its last token to the next step
as root ("Medusa 深读": greedy acceptance keeps the longest prefix that agrees
with the base model)."""

import numpy as np
import pytest

from oracle import generate as OG
from workloads import cartesian_ranks, planted_inputs

A = np.array([[0.70, 0.15, 0.05], [0.60, 0.15, 0.05], [0.50, 0.15, 0.05],
              [0.45, 0.10, 0.05], [0.40, 0.10, 0.05]])
SPEC = cartesian_ranks((3, 2, 2, 1, 1))
KW = dict(H=4, Dh=128, s_max=3, mode="greedy", tau=1.0, eps=0.09, delta=0.3, theta=10000.0,
          bf16=True)


def predicted_depth(spec, true_rank, t):
    paths = {tuple(int(x) for x in row if x >= 0) for row in spec}
    d = 0
    while d < true_rank.shape[0] and tuple(int(true_rank[j, t]) for j in range(d + 1)) in paths:
        d += 1
    return d


@pytest.mark.parametrize("spec", [SPEC, np.array([[0, -1, -1, -1, -1], [0, 0, -1, -1, -1],
                                                  [0, 0, 0, -1, -1]], dtype=np.int32)])
def test_planted_loop_follows_the_language(spec):
    n = 10
    inp = planted_inputs(A, spec, n_steps=n)
    r = OG.generate(inp, n, **KW)
    pi = inp["pi"]
    t_last = int(np.argmax(inp["h"][0]))
    root = int(inp["root"][0])
    kv = int(inp["kv_len"][0])
    for i in range(n):
        a = int(r["accept_len"][i, 0])
        toks = r["out_tokens"][i, 0]
        assert toks[0] == root
        for j in range(a):
            assert toks[j + 1] == pi[toks[j]]
        assert np.all(toks[a + 1:] == -1)
        assert a == predicted_depth(spec, inp["true_rank"], t_last)
        kv += a + 1
        t_last = int(toks[a])
        root = int(pi[t_last])
    assert int(r["root"][0]) == root
    assert int(r["kv_len"][0]) == kv
    assert int(np.argmax(r["h"][0])) == t_last
    assert r["accept_len"].sum() > 0
