"""GPTQ column loop, RTN baseline, reconstruction error, replay (oracle, test infrastructure only).

The column loop follows "GPTQ deep dive" §3.1 step 3 and §2.4:
* columns are taken in a fixed order, left to right in processing order
  (§2.4, first acceleration; with desc_act the order is by descending
  Hessian diagonal, §3.3);
* the columns are cut into blocks of ``block_size`` (128 by default, §3.1
  step 3; a multiple of group_size per "AWQ, MinMax, GPTQ calibration in
  Model Optimizer" §4);
* inside a block, each column is quantized with its group's scale and
  zero-point, computed when the group's first column is reached from the
  current, already-compensated weights; the column's error is pushed onto the
  not-yet-quantized columns of the block at once (§2.2: the quantization error
  of one weight is compensated by the others through the inverse Hessian);
* after the block, all later columns receive the block's accumulated errors
  in one batched product (§2.4, second acceleration, lazy batch update);
* the inverse Hessian enters through U, the upper Cholesky factor of H_d^-1
  (§2.4, third acceleration; §3.1 step 2).

Readings of the pages adopted here:
* §2.2 prints the compensation with numerator w_q, which is the pruning form;
  for quantization the numerator is the quantization error w_q - quant(w_q)
  (the surrounding text speaks of compensating the quantization error).
* "accumulate errors inside the block, then update once" (§2.4) is read as:
  errors update the rest of the block immediately; only columns beyond the
  block are deferred.  This is the reading under which the result does not
  depend on the block size.

* Static groups (a variant the pages do not describe; the plain reading of
  the name): every group's parameters are computed once, before the loop,
  from the original weights, for groups of consecutive original columns.
* A group spanning several blocks (group_size a multiple of block_size) is
  read as block_size = group_size ("AWQ, MinMax, GPTQ calibration in Model
  Optimizer" §4): its parameters come from the current values of its columns
  at its first column, which is a block start.

``gptq_obs_literal`` is a second, independent route: it keeps H_d^-1
explicitly and applies the §2.2 compensation formula column by column, with
the inverse downdated after each column; it shares only the quantizer.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .quantizer import dequantize, f32, group_params, pre_round_value, quantize_codes


@dataclasses.dataclass
class GPTQResult:
    codes: np.ndarray     # [m, n] integral fp64 -> original column order
    scales: np.ndarray    # [m, ngroups] processing-order groups
    zeros: np.ndarray     # [m, ngroups]
    g_idx: np.ndarray     # [n] group of each original column
    perm: np.ndarray      # [n]
    E: np.ndarray         # [m, n] scaled errors e_c in processing order
    codes_proc: np.ndarray  # [m, n] codes in processing order


def _ngroups(n: int, G: int) -> int:
    return 1 if G <= 0 else (n + G - 1) // G


def _check_grouping(n: int, G: int, B: int) -> None:
    if B <= 0:
        raise ValueError("block_size must be positive")
    if G > 0 and B % G != 0 and G % B != 0:
        raise ValueError("block_size must be a multiple of group_size (or group_size of "
                         "block_size, which computes the same result as block_size = group_size)")


def gptq_quantize(W: np.ndarray, U: np.ndarray, bits: int, group_size: int,
                  block_size: int = 128, perm: Optional[np.ndarray] = None,
                  dead: Optional[np.ndarray] = None, sym: bool = False,
                  static_groups: bool = False, exact: bool = False) -> GPTQResult:
    """Blocked GPTQ of W [m, n] (original column order) with U from ``prepare``.

    ``static_groups``: the group parameters are computed once, before the loop,
    from the original W (dead columns zeroed), for groups of consecutive
    ORIGINAL columns; a column uses the parameters of its original group, so
    with desc_act g_idx stays c // G.  Otherwise (dynamic) a group is G
    consecutive processing positions and its parameters come from the current,
    compensated values when its first column is reached.  A group larger than
    the block (G a multiple of B) starts at a block start, where every earlier
    column's error has been applied to all later columns, so its parameters are
    those block_size = G would give.

    ``exact``: the quantizer's decisions (range, scale, zero-point, codes) in
    plain fp64 instead of the fp32 decision precision."""
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    G, B = group_size, block_size
    _check_grouping(n, G, B)
    if perm is None:
        perm = np.arange(n)
    Wp = W[:, perm].copy()
    if dead is not None:
        Wp[:, np.asarray(dead)[perm]] = 0.0
    ng = _ngroups(n, G)
    scales = np.zeros((m, ng))
    zeros = np.zeros((m, ng))
    Q = np.zeros((m, n))
    Eall = np.zeros((m, n))
    if G <= 0:  # one group per row, taken from the whole (unmodified) row
        scale, zero = group_params(Wp, bits, sym, exact)
        scales[:, 0], zeros[:, 0] = scale, zero
    elif static_groups:
        W0 = W.copy()
        if dead is not None:
            W0[:, np.asarray(dead)] = 0.0
        for g in range(ng):
            scales[:, g], zeros[:, g] = group_params(W0[:, g * G:(g + 1) * G], bits, sym, exact)
    for i in range(0, n, B):
        i1 = min(i + B, n)
        W1 = Wp[:, i:i1].copy()
        E = np.zeros((m, i1 - i))
        for j in range(i1 - i):
            c = i + j
            if G > 0 and static_groups:
                g = int(perm[c]) // G
                scale, zero = scales[:, g], zeros[:, g]
            elif G > 0 and c % G == 0:
                glen = min(G, n - c)
                cur = W1[:, j:j + glen] if G <= B else Wp[:, c:c + glen]  # c == i when G > B
                scale, zero = group_params(cur, bits, sym, exact)
                scales[:, c // G], zeros[:, c // G] = scale, zero
            w = W1[:, j]
            q = quantize_codes(w, scale, zero, bits, exact)
            e = (w - dequantize(q, scale, zero)) / U[c, c]
            W1[:, j + 1:] -= np.outer(e, U[c, c + 1:i1])
            E[:, j] = e
            Q[:, c] = q
        Eall[:, i:i1] = E
        if i1 < n:
            Wp[:, i1:] -= E @ U[i:i1, i1:]
    codes = np.empty_like(Q)
    codes[:, perm] = Q
    g_idx = np.empty(n, dtype=np.int64)
    if G > 0 and static_groups:
        g_idx[:] = np.arange(n) // G
    else:
        g_idx[perm] = (np.arange(n) // G) if G > 0 else 0
    return GPTQResult(codes=codes, scales=scales, zeros=zeros, g_idx=g_idx, perm=perm,
                      E=Eall, codes_proc=Q)


def gptq_obs_literal(W: np.ndarray, Hd: np.ndarray, bits: int, group_size: int,
                     perm: Optional[np.ndarray] = None, sym: bool = False,
                     exact: bool = False):
    """Fixed-order OBS route: explicit H_d^-1, compensation and downdate per column.

    ``Hd`` is the damped Hessian in processing order.  Returns (codes in original
    order, scales, zeros).  O(n^3); meant for small n.
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    G = group_size
    if perm is None:
        perm = np.arange(n)
    Wp = W[:, perm].copy()
    Hinv = np.linalg.inv(np.asarray(Hd, dtype=np.float64))
    ng = _ngroups(n, G)
    scales = np.zeros((m, ng))
    zeros = np.zeros((m, ng))
    Q = np.zeros((m, n))
    if G <= 0:
        scale, zero = group_params(Wp, bits, sym, exact)
        scales[:, 0], zeros[:, 0] = scale, zero
    for c in range(n):
        if G > 0 and c % G == 0:
            scale, zero = group_params(Wp[:, c:min(c + G, n)], bits, sym, exact)
            scales[:, c // G], zeros[:, c // G] = scale, zero
        q = quantize_codes(Wp[:, c], scale, zero, bits, exact)
        err = Wp[:, c] - dequantize(q, scale, zero)
        d = Hinv[c, c]
        # compensation: delta_F = -(err / [H^-1]_cc) * [H^-1]_{c, F}
        Wp[:, c + 1:] -= np.outer(err / d, Hinv[c, c + 1:])
        Wp[:, c] = dequantize(q, scale, zero)
        # remove column c from the inverse of the remaining sub-Hessian
        Hinv = Hinv - np.outer(Hinv[:, c], Hinv[c, :]) / d
        Q[:, c] = q
    codes = np.empty_like(Q)
    codes[:, perm] = Q
    return codes, scales, zeros


def rtn_minmax(W: np.ndarray, bits: int, group_size: int, sym: bool = False,
               exact: bool = False):
    """Round-to-nearest with group min-max parameters from the original weights.

    The GPTQ loop with no compensation: "GPTQ deep dive" §1.2 (RTN rounds each
    weight independently) and "Calibration algorithms guide" §2.2 (group-wise
    min-max).  Groups are consecutive columns in original order.
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    G = group_size if group_size > 0 else n
    ng = (n + G - 1) // G
    codes = np.zeros((m, n))
    scales = np.zeros((m, ng))
    zeros = np.zeros((m, ng))
    for g in range(ng):
        c0, c1 = g * G, min((g + 1) * G, n)
        scale, zero = group_params(W[:, c0:c1], bits, sym, exact)
        scales[:, g], zeros[:, g] = scale, zero
        codes[:, c0:c1] = quantize_codes(W[:, c0:c1], scale[:, None], zero[:, None], bits, exact)
    return codes, scales, zeros


def dequant_layer(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                  g_idx: np.ndarray) -> np.ndarray:
    """Dequantized weights in original column order (gathering each column's group)."""
    g = np.asarray(g_idx)
    return dequantize(codes, scales[:, g], zeros[:, g])


def recon_error_from_H(W: np.ndarray, Wq: np.ndarray, H: np.ndarray) -> float:
    """||WX - W_qX||_F^2 = 1/2 * sum_r delta_r^T H delta_r with H = 2XX^T (undamped).

    The layer objective of "LLM quantization principles" §3.1; W, Wq and H share
    one column order.
    """
    D = np.asarray(W, np.float64) - np.asarray(Wq, np.float64)
    return 0.5 * float(np.sum((D @ np.asarray(H, np.float64)) * D))


def recon_error_direct(W: np.ndarray, Wq: np.ndarray, X_tokens: np.ndarray) -> float:
    """||WX - W_qX||_F^2 computed from the activations X_tokens [tokens, n]."""
    D = np.asarray(W, np.float64) - np.asarray(Wq, np.float64)
    Y = D @ np.asarray(X_tokens, np.float64).T
    return float(np.sum(Y * Y))


@dataclasses.dataclass
class ReplayReport:
    n_codes: int
    mismatches: int
    ties: int
    hard: int
    zero_mismatches: int
    zero_ties: int
    zero_hard: int
    scale_max_rel: float
    row_err: np.ndarray


def replay_check(W: np.ndarray, U: np.ndarray, bits: int, group_size: int, block_size: int,
                 perm: Optional[np.ndarray], dead: Optional[np.ndarray],
                 codes_proc: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                 tau: float = 1e-3, sym: bool = False,
                 static_groups: bool = False, exact: bool = False) -> ReplayReport:
    """Validate a candidate result column by column against the oracle's own loop.

    At a rounding tie both neighbours are correct, and everything downstream
    depends on which was taken.  So the loop runs on the oracle's arithmetic but
    follows the candidate's choices: at each column the candidate code must be
    the oracle's rounding of its own pre-rounding value, or, when that value lies
    within ``tau`` (in quantization steps) of a rounding boundary, the other
    neighbour.  Any other disagreement is "hard".  Group zero-points are checked
    the same way; scales must agree to ``scale_max_rel``, which is reported.
    ``exact``: the oracle's side of every decision in plain fp64.
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    G, B = group_size, block_size
    maxq = float(2 ** bits - 1)
    if perm is None:
        perm = np.arange(n)
    Wp = W[:, perm].copy()
    if dead is not None:
        Wp[:, np.asarray(dead)[perm]] = 0.0
    cq = np.asarray(codes_proc, dtype=np.float64)
    mism = ties = hard = 0
    zmis = zties = zhard = 0
    smax = 0.0
    row_err = np.zeros(m)

    def take_params(vals, gidx):
        nonlocal zmis, zties, zhard, smax
        s_o, z_o = group_params(vals, bits, sym, exact)
        s_c = np.asarray(scales[:, gidx], np.float64)
        z_c = np.asarray(zeros[:, gidx], np.float64)
        smax = max(smax, float(np.max(np.abs(s_c - s_o) / np.abs(s_o))))
        bad = z_c != z_o
        if np.any(bad) and not sym:
            rd = f32 if not exact else (lambda x: np.asarray(x, dtype=np.float64))
            v32 = rd(vals)
            xmin = np.minimum(v32.min(axis=1), 0.0)
            xmax = np.maximum(v32.max(axis=1), 0.0)
            flat = xmin == xmax
            xmin = np.where(flat, -1.0, xmin)
            span = rd(np.where(flat, 1.0, xmax) - xmin)
            pre = rd(rd(-xmin * maxq) / span)
            frac = np.abs(pre - np.floor(pre) - 0.5)
            tie = bad & (frac < tau) & (np.abs(z_c - z_o) == 1)
            zmis += int(bad.sum())
            zties += int(tie.sum())
            zhard += int((bad & ~tie).sum())
        elif np.any(bad):
            zmis += int(bad.sum())
            zhard += int(bad.sum())
        return s_c, z_c

    if G <= 0:
        scale, zero = take_params(Wp, 0)
    elif static_groups:
        W0 = W.copy()
        if dead is not None:
            W0[:, np.asarray(dead)] = 0.0
        for g in range((n + G - 1) // G):
            take_params(W0[:, g * G:(g + 1) * G], g)
    for i in range(0, n, B):
        i1 = min(i + B, n)
        W1 = Wp[:, i:i1].copy()
        E = np.zeros((m, i1 - i))
        for j in range(i1 - i):
            c = i + j
            if G > 0 and static_groups:
                g = int(perm[c]) // G
                scale = np.asarray(scales[:, g], np.float64)
                zero = np.asarray(zeros[:, g], np.float64)
            elif G > 0 and c % G == 0:
                cur = W1[:, j:j + min(G, n - c)] if G <= B else Wp[:, c:c + min(G, n - c)]
                scale, zero = take_params(cur, c // G)
            w = W1[:, j]
            q_o = quantize_codes(w, scale, zero, bits, exact)
            q_c = cq[:, c]
            bad = q_c != q_o
            if np.any(bad):
                pre = pre_round_value(w, scale, exact)
                frac = np.abs(pre - np.floor(pre) - 0.5)
                tie = bad & (frac < tau) & (np.abs(q_c - q_o) == 1)
                mism += int(bad.sum())
                ties += int(tie.sum())
                hard += int((bad & ~tie).sum())
            e = (w - dequantize(q_c, scale, zero)) / U[c, c]
            row_err += e * e
            W1[:, j + 1:] -= np.outer(e, U[c, c + 1:i1])
            E[:, j] = e
        if i1 < n:
            Wp[:, i1:] -= E @ U[i:i1, i1:]
    return ReplayReport(n_codes=m * n, mismatches=mism, ties=ties, hard=hard,
                        zero_mismatches=zmis, zero_ties=zties, zero_hard=zhard,
                        scale_max_rel=smax, row_err=row_err)
