"""Damping, column order and the inverse-Hessian factor (oracle, test infrastructure only).

Steps, in the order of "GPTQ deep dive" §3.1 (steps 1-2) and §3.3:
1. H = 2S.
2. Dead columns (H_ii == 0, a channel that is never active): H_ii := 1 and the
   matching weight column is zeroed before quantization.  The pages are silent
   here; the rule keeps the damped matrix positive definite.
3. desc_act ("GPTQ deep dive" §3.3; "Calibration algorithms guide" §2.3):
   process columns by descending Hessian diagonal.  Stable sort, so equal keys
   keep ascending original index.  H is permuted symmetrically.
4. lambda = perc_damp * mean(diag H) ("GPTQ deep dive" §3.3, damp_percent
   default 0.01; "AWQ, MinMax, GPTQ calibration in Model Optimizer" §4,
   perc_damp 0.01), H_d = H + lambda*I.
5. The column loop needs the upper Cholesky factor U of H_d^-1
   (H_d^-1 = U^T U): "GPTQ deep dive" §2.4 replaces repeated inversion by a
   Cholesky factorization and §3.1 step 2 factors the Hessian.  The oracle
   takes the textbook route with LAPACK: Cholesky-factor H_d, solve for
   H_d^-1, then take the upper Cholesky factor of H_d^-1.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import scipy.linalg as sla


@dataclasses.dataclass
class Prepared:
    U: np.ndarray        # [n, n] upper, H_d^-1 = U^T U, processing order
    perm: np.ndarray     # [n] processing position k -> original column perm[k]
    dead: np.ndarray     # [n] bool, original column order
    lam: float           # damping added to the diagonal
    H: np.ndarray        # [n, n] undamped H after the dead fix, processing order
    Hd: np.ndarray       # [n, n] damped H, processing order


class NotPositiveDefinite(ValueError):
    pass


def prepare(S: np.ndarray, perc_damp: float = 0.01, desc_act: bool = False,
            order: np.ndarray | None = None) -> Prepared:
    """``order``: with desc_act, an externally chosen processing order to use instead
    of the argsort.  Keys that differ by less than the accumulation error of S may be
    ordered either way (both orders are correct); a caller that has checked an order
    with ``check_descending_order`` passes it here so the rest of the computation
    follows that choice."""
    S = np.asarray(S, dtype=np.float64)
    n = S.shape[0]
    H = 2.0 * S
    d = np.diag(H).copy()
    dead = d == 0.0
    H[dead, dead] = 1.0
    if desc_act and order is not None:
        perm = np.asarray(order, dtype=np.int64)
        if not np.array_equal(np.sort(perm), np.arange(n)):
            raise ValueError("order is not a permutation")
    elif desc_act:
        perm = np.argsort(-np.diag(H), kind="stable")
    else:
        perm = np.arange(n)
    H = H[np.ix_(perm, perm)]
    lam = float(perc_damp) * float(np.mean(np.diag(H)))
    Hd = H + lam * np.eye(n)
    try:
        cf = sla.cho_factor(Hd, lower=True)
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from exc
    Hinv = sla.cho_solve(cf, np.eye(n))
    U = sla.cholesky(Hinv, lower=False)
    return Prepared(U=U, perm=perm, dead=dead, lam=lam, H=H, Hd=Hd)


def check_descending_order(order: np.ndarray, diag: np.ndarray, rel_tol: float) -> int:
    """Validate ``order`` as a descending order of ``diag`` up to ``rel_tol``.

    Every key must be at most rel_tol * max|diag| above the smallest key placed
    before it.  Returns the number of positions at which ``order`` differs from the
    exact stable order; raises ValueError if ``order`` is not a permutation or
    places a key above an earlier one by more than the tolerance.
    """
    order = np.asarray(order, dtype=np.int64)
    n = diag.shape[0]
    if not np.array_equal(np.sort(order), np.arange(n)):
        raise ValueError("not a permutation")
    d = np.asarray(diag, dtype=np.float64)[order]
    tol = rel_tol * float(np.max(np.abs(diag))) if n else 0.0
    if n > 1:
        rise = d[1:] - np.minimum.accumulate(d[:-1])  # must be <= 0 for a descending order
        if np.any(rise > tol):
            k = int(np.argmax(rise)) + 1
            raise ValueError(f"order raises key at position {k} by {rise[k - 1]:.3e} > {tol:.3e}")
    exact = np.argsort(-np.asarray(diag, dtype=np.float64), kind="stable")
    return int(np.sum(order != exact))
