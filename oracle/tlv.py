"""Two-level verification (TLV) -- oracle.

Source: SpecPilot summary (onedev.kr), section 무엇과 다른가: a Q pass over
the draft tree, run on the 8-bit leading view of the W12 records, yields the
matched path and a bonus token; a subtree drafted again from the end of that
path is attached, and the resulting tree (32 nodes) is checked by one exact
pass.  Section 전제와 한계 gives its cost: the Q pass takes 0.80-0.88 of a
step, so the exact pass must accept nearly twice the tokens to break even.

Readings of what the page leaves open (the plainest the rest supports):

* the Q pass is the ordinary tree-verification pass of ``model.verify`` with
  every W12 weight (the LM head included) seen through ``w12.decode_hi8``;
  its keys and values are scratch and never committed;
* the exact tree is the Q pass's matched path (root first, as a chain), then
  the Q bonus token as a child of the path's last node, then the re-drafted
  subtree below the bonus node -- node order: path, bonus, subtree in its own
  topological order; ``subtree_parents`` are local to the subtree (its node
  0 is the bonus node itself, parent -1);
* the exact pass is ``model.verify`` on that tree; what it accepts is what
  the step emits, so the emitted tokens are the exact greedy stream whatever
  the Q pass got wrong.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from . import accept as _accept
from . import model as _model


def exact_tree(q_path: Sequence[int], draft_tokens: Sequence[int], q_bonus: int,
               subtree_parents: Sequence[int], subtree_tokens: Sequence[int]):
    """Tokens and parents of the tree the exact pass checks."""
    path = [int(v) for v in q_path]
    sp = np.asarray(subtree_parents, dtype=np.int64)
    st = np.asarray(subtree_tokens, dtype=np.int64)
    if len(sp) < 1 or sp[0] != -1 or int(st[0]) != int(q_bonus):
        raise ValueError("the subtree's node 0 is the bonus token, with parent -1")
    _accept.validate_tree(sp)
    a = len(path)  # nodes of the matched path (root included)
    tokens = [int(draft_tokens[v]) for v in path] + [int(t) for t in st]
    parents = [-1] + list(range(a - 1))  # the path as a chain
    parents += [a - 1] + [a + int(p) for p in sp[1:]]  # bonus under the path's end, subtree below it
    return np.asarray(tokens, dtype=np.int64), np.asarray(parents, dtype=np.int64)


def tlv_step(model_q: _model.OracleModel, model_exact: _model.OracleModel, cache: _model.KVCache,
             ctx_len: int, tokens: Sequence[int], parents: Sequence[int], redraft) -> dict:
    """One TLV step.  ``redraft(q_path, q_bonus) -> (subtree_parents,
    subtree_tokens)`` stands in for the drafter."""
    q = _model.verify(model_q, cache, ctx_len, tokens, parents)
    sp, st = redraft(q["path"], q["bonus"])
    et, ep = exact_tree(q["path"], tokens, q["bonus"], sp, st)
    ex = _model.verify(model_exact, cache, ctx_len, et, ep)
    return {"q": q, "tokens": et, "parents": ep, "exact": ex}
