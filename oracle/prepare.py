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


def prepare(S: np.ndarray, perc_damp: float = 0.01, desc_act: bool = False) -> Prepared:
    S = np.asarray(S, dtype=np.float64)
    n = S.shape[0]
    H = 2.0 * S
    d = np.diag(H).copy()
    dead = d == 0.0
    H[dead, dead] = 1.0
    if desc_act:
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
