"""LM head on INT8 weights with a Cauchy-Schwarz certified candidate filter
(oracle).

Source: SpecPilot summary (onedev.kr), section 무엇과 다른가: on one GPU the
LM head filters candidate tokens with INT8 weights and a Cauchy-Schwarz error
bound, and the exact argmax is kept; on another GPU that filter is slower
than the W12 head.  The page gives no format details; the readings below
are the plainest that make the filter certify the exact argmax.

* Weights per vocabulary row v (bf16 ``W_v``, ``k_in`` columns): the row's
  ``n_esc`` (8) largest magnitudes (ties to the smaller column) are escapes;
  the scale ``s_v = fp32(t_v / 127)`` with ``t_v`` the largest remaining
  magnitude (``s_v = 1`` when that is 0); every other weight is
  ``q = clip(rint(fp32(w) / s_v), -127, 127)`` (fp32 division, ties to even).
  An escape is carried as ``bf16(fp32(w) / s_v)`` in the same units.  So the
  row stands for ``W^_v = s_v * B_v`` with ``B_v`` the int8 values and the
  rounded escapes.  Keeping the largest magnitudes out of the scale follows
  W12's own escapes: on weights with rare large outliers a scale set by the
  outliers leaves most of the vocabulary as candidates.
* ``r_v = ||W_v - W^_v||_2``, computed exactly and stored as fp32 rounded up.
* Approximate logits ``a_v = f . W^_v``; by Cauchy-Schwarz
  ``|f . W_v - a_v| <= ||f||_2 r_v = b_v``.
* Certified candidates: with ``tau = max_v (a_v - b_v)``, every v with
  ``a_v + b_v >= tau``.  The exact argmax u has ``f.W_u >= tau`` (it beats
  the row attaining tau, whose exact logit is at least tau) and
  ``f.W_u <= a_u + b_u``, so it is a candidate.
* The head's result is the argmax of the exact logits over the candidates,
  ties to the smallest token id: the argmax of the whole exact row.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .bf16 import from_bits, round_bf16

N_ESC = 8


@dataclass
class I8Head:
    q: np.ndarray        # int8   [V, k]  (0 at escaped columns)
    scale: np.ndarray    # fp32   [V]
    esc_col: np.ndarray  # int64  [V, n_esc]
    esc_val: np.ndarray  # fp64   [V, n_esc]  bf16 values of w / s
    r: np.ndarray        # fp32   [V]   ||W_v - W^_v||_2, rounded up

    def dequant(self) -> np.ndarray:
        """B_v (fp64): int8 values with the escapes in place."""
        b = self.q.astype(np.float64)
        rows = np.arange(b.shape[0])[:, None]
        b[rows, self.esc_col] = self.esc_val
        return b


def encode(w_bits: np.ndarray, n_esc: int = N_ESC) -> I8Head:
    w = from_bits(np.asarray(w_bits, dtype=np.uint16))
    V, k = w.shape
    n_esc = min(n_esc, k)
    mag = np.abs(w)
    # order by magnitude, largest first, ties to the smaller column
    order = np.lexsort((np.broadcast_to(np.arange(k), (V, k)), -mag), axis=1)
    esc_col = np.sort(order[:, :n_esc], axis=1)
    rows = np.arange(V)[:, None]
    t = mag[rows, order[:, n_esc:n_esc + 1]][:, 0] if n_esc < k else np.zeros(V)
    scale = (t.astype(np.float32) / np.float32(127.0)).astype(np.float32)
    scale[scale == 0] = np.float32(1.0)
    ratio = (w.astype(np.float32) / scale[:, None]).astype(np.float32)
    q = np.clip(np.rint(ratio), -127, 127)
    q[rows, esc_col] = 0
    esc_val = round_bf16(ratio[rows, esc_col].astype(np.float64))
    head = I8Head(q.astype(np.int8), scale, esc_col.astype(np.int64), esc_val, np.zeros(V, np.float32))
    err = w - scale.astype(np.float64)[:, None] * head.dequant()
    r = np.sqrt(np.sum(err * err, axis=1))
    r32 = r.astype(np.float32)
    up = r32.astype(np.float64) < r
    r32[up] = np.nextafter(r32[up], np.float32(np.inf))
    head.r = r32
    return head


def approx_logits(f: np.ndarray, head: I8Head) -> np.ndarray:
    """a = f . W^^T, fp64, ``f [m, k]``."""
    return (np.asarray(f, np.float64) @ head.dequant().T) * head.scale.astype(np.float64)[None, :]


def candidates(f: np.ndarray, head: I8Head) -> np.ndarray:
    """Boolean ``[m, V]``: the certified candidate set of every row."""
    a = approx_logits(f, head)
    b = np.linalg.norm(np.asarray(f, np.float64), axis=1)[:, None] * head.r.astype(np.float64)[None, :]
    tau = np.max(a - b, axis=1, keepdims=True)
    return a + b >= tau


def argmax(f: np.ndarray, head: I8Head, w_bits: np.ndarray) -> np.ndarray:
    """Exact greedy token of every row: the exact logits of the candidates only."""
    cand = candidates(f, head)
    w = from_bits(np.asarray(w_bits, dtype=np.uint16))
    f = np.asarray(f, np.float64)
    out = np.empty(f.shape[0], dtype=np.int64)
    for i in range(f.shape[0]):
        ids = np.flatnonzero(cand[i])
        ex = w[ids] @ f[i]
        out[i] = ids[int(np.argmax(ex))]  # ids ascending: the first maximum is the smallest id
    return out
