"""Two-level verification (TLV) on the device model.

SpecPilot summary (onedev.kr), section 무엇과 다른가: a Q pass over the draft
tree on the 8-bit leading view of the W12 records gives the matched path and
a bonus token; a subtree drafted again from the end of that path is attached
and the whole tree (32 nodes) goes through one exact pass.  Section 전제와
한계: the Q pass costs 0.80-0.88 of a step.

Both passes are ``verify_step`` (the Q pass on ``DeviceModel.q_plan``, whose
weights are the packed 8-bit views, without commit; the exact pass on
``DeviceModel.plan``, with commit).  Between them the host reads the Q
pass's path and bonus and assembles the exact tree: the matched path as a
chain (root first), the bonus token as the child of its last node, then the
re-drafted subtree below the bonus (its parents local to the subtree, its
node 0 being the bonus itself).  The drafter is the caller's ``redraft``.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Sequence, Tuple

import numpy as np
import torch

from . import VerifyResult, verify_step


def exact_tree(q_path: Sequence[int], draft_tokens: Sequence[int], q_bonus: int, sub_parents: Sequence[int],
               sub_tokens: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """``(tokens, parents)`` int32 of the tree the exact pass checks."""
    path = np.asarray(q_path, dtype=np.int64)
    sp = np.asarray(sub_parents, dtype=np.int64)
    st = np.asarray(sub_tokens, dtype=np.int64)
    if sp.size < 1 or sp[0] != -1 or int(st[0]) != int(q_bonus) or st.size != sp.size:
        raise ValueError("the subtree's node 0 must be the bonus token with parent -1")
    if np.any(sp[1:] < 0) or np.any(sp[1:] >= np.arange(1, sp.size)):
        raise ValueError("subtree parents must precede their children")
    a = path.size
    tok = np.concatenate([np.asarray(draft_tokens, dtype=np.int64)[path], st])
    par = np.concatenate([np.arange(-1, a - 1), [a - 1], a + sp[1:]])
    return tok.astype(np.int32), par.astype(np.int32)


@dataclass
class TlvResult:
    q: VerifyResult          # the Q pass over the draft tree
    tokens: np.ndarray       # the exact tree
    parents: np.ndarray
    exact: VerifyResult      # the exact pass over it (committed when asked)


def tlv_step(dm, ctx_len: int, tokens: torch.Tensor, parents: torch.Tensor,
             redraft: Callable[[np.ndarray, int], Tuple[Sequence[int], Sequence[int]]], commit: bool = True,
             want_logits: bool = False) -> TlvResult:
    """One TLV step on ``dm`` (built ``with_hi8``) after ``ctx_len`` committed
    tokens; ``tokens``/``parents`` (device int32) are the draft tree."""
    if dm.q_plan is None:
        raise ValueError("the model has no 8-bit views: build it with with_hi8=True")
    q = verify_step(dm.q_plan, ctx_len, tokens, parents, commit=False, want_logits=want_logits)
    a = int(q.n_accepted.item())  # the one readback between the passes
    q_path = q.path[: a + 1].cpu().numpy()
    q_bonus = int(q.bonus.item())
    sp, st = redraft(q_path, q_bonus)
    et, ep = exact_tree(q_path, tokens.cpu().numpy(), q_bonus, sp, st)
    dev = tokens.device
    ex = verify_step(dm.plan, ctx_len, torch.as_tensor(et, device=dev), torch.as_tensor(ep, device=dev),
                     commit=commit, want_logits=want_logits)
    return TlvResult(q, et, ep, ex)
