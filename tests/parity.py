"""Comparison rules between a result under test and the oracle.

* Logits: per row, ``max_t |g_t - r_t| / max_t |r_t| <= 2e-3`` (bf16 inputs and
  outputs, fp32 accumulation).  Through the composed pass, whose bf16
  rounding points let an fp32-vs-fp64 rounding flip of one activation move
  a logit by more (SpecPilot summary, section 전제와 한계: reduction order
  may flip near-ties), every row may deviate by max(2e-3, 1.5 x env), where
  env is the largest deviation of any row across fp32 evaluations of the
  same definition with other summation orders (tests/fp32_reference.py),
  and never by more than ROW_TOL_CAP.  A row's own envelope is not used as
  its bound: row deviations are heavy-tailed (a rare flip times an outlier
  weight), so a few evaluations estimate one row's spread badly
  (tests/test_oracle_fp32_noise.py shows a fresh fp32 evaluation failing
  such a per-row bound on several percent of rows).
* Greedy tokens: a row is *decidable* when the oracle's top-2 margin exceeds
  twice the row's measured error ``delta = max_t |g_t - r_t|``.  Then no error
  of that size can change the argmax, so the two argmaxes must agree.  Rows
  that are not decidable are near-ties, which a different reduction order may
  flip (SpecPilot summary, section 전제와 한계).
* Accepted paths: the result's own path must follow exactly from its own
  greedy tokens, and it must equal the oracle's path up to the first node on
  the oracle path that is not decidable.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

LOGIT_TOL = 2e-3
# Hard ceiling of the per-row end-to-end tolerance, whatever the envelope.
ROW_TOL_CAP = 2e-2
ENV_FACTOR = 1.5


def row_max_abs_rel(g: np.ndarray, r: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return np.max(np.abs(g - r), axis=-1) / np.maximum(np.max(np.abs(r), axis=-1), 1e-300)


def row_delta(g: np.ndarray, r: np.ndarray) -> np.ndarray:
    return np.max(np.abs(np.asarray(g, np.float64) - np.asarray(r, np.float64)), axis=-1)


def top2_margin(r: np.ndarray) -> np.ndarray:
    part = np.partition(np.asarray(r, np.float64), -2, axis=-1)
    return part[..., -1] - part[..., -2]


def decidable_rows(g: np.ndarray, r: np.ndarray) -> np.ndarray:
    return top2_margin(r) > 2.0 * row_delta(g, r)


def row_tolerances(env_rows: np.ndarray, floor: float = LOGIT_TOL, factor: float = ENV_FACTOR,
                   cap: float = ROW_TOL_CAP) -> np.ndarray:
    """The bound of every row of one comparison: max(floor, factor x the
    largest deviation over the rows' envelopes), at most ``cap``."""
    env = np.asarray(env_rows, np.float64)
    t = min(cap, max(floor, factor * float(env.max()) if env.size else floor))
    return np.full(env.shape, t)


def check_logits(g: np.ndarray, r: np.ndarray, tol=LOGIT_TOL) -> dict:
    """``tol``: one bound for every row, or an array of per-row bounds."""
    err = row_max_abs_rel(g, r)
    tol = np.broadcast_to(np.asarray(tol, np.float64), err.shape)
    dec = decidable_rows(g, r)
    am_g = np.argmax(g, axis=-1)
    am_r = np.argmax(r, axis=-1)
    bad_argmax = np.flatnonzero(dec & (am_g != am_r))
    return {
        "max_abs_rel": float(err.max()) if err.size else 0.0,
        "logits_ok": bool(np.all(err <= tol)),
        "bad_rows": np.flatnonzero(err > tol).tolist(),
        "row_err": err,
        "frac_above_2e-3": float(np.mean(err > LOGIT_TOL)) if err.size else 0.0,
        "decidable": dec,
        "undecidable_frac": float(1.0 - dec.mean()) if dec.size else 0.0,
        "argmax_ok": bad_argmax.size == 0,
        "bad_argmax_rows": bad_argmax.tolist(),
    }


def row_report(chk: dict, env_rows: np.ndarray, tol_rows: np.ndarray) -> str:
    """One line on the per-row comparison: the largest error, the share of rows
    above the plain 2e-3, and the largest error as a share of its row's bound."""
    err = chk["row_err"]
    env = np.asarray(env_rows, np.float64)
    return (f"max_abs_rel={err.max():.2e} rows>2e-3={chk['frac_above_2e-3']:.3f} "
            f"max_env={env.max():.2e} tol={np.max(tol_rows):.2e} max_err/tol={np.max(err / tol_rows):.2f} "
            f"rows err>own env={np.mean(err > env):.3f} undecidable={chk['undecidable_frac']:.3f}")


def path_prefix_ok(path_g: Sequence[int], path_r: Sequence[int], decidable: np.ndarray) -> bool:
    """Paths agree up to (and including) the first undecidable node on the oracle path."""
    for j, node in enumerate(path_r):
        if j >= len(path_g) or path_g[j] != node:
            return False
        if not decidable[node]:
            return True
    return len(path_g) == len(path_r)


def accepted_flags(argmax: Sequence[int], tokens: Sequence[int], parents: Sequence[int]) -> np.ndarray:
    n = len(parents)
    ok = np.zeros(n, dtype=bool)
    ok[0] = True
    for i in range(1, n):
        ok[i] = ok[parents[i]] and int(tokens[i]) == int(argmax[parents[i]])
    return ok


def acceptance_ok(argmax_g, argmax_r, tokens, parents, decidable: np.ndarray) -> bool:
    """Acceptance of a node is fixed by the greedy tokens of its strict ancestors;
    where those are all decidable, both sides must agree on it."""
    n = len(parents)
    determined = np.ones(n, dtype=bool)
    for i in range(1, n):
        p = parents[i]
        determined[i] = determined[p] and bool(decidable[p])
    a_g = accepted_flags(argmax_g, tokens, parents)
    a_r = accepted_flags(argmax_r, tokens, parents)
    return bool(np.all(a_g[determined] == a_r[determined]))
