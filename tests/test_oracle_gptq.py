"""Pins for the oracle's GPTQ column loop, RTN and reconstruction error (CPU only)."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from oracle.quantizer import f32


def _layer(m, n, tokens, seed=0, outliers=True, wscale=0.02):
    rng = np.random.default_rng(seed)
    W = f32(rng.standard_normal((m, n)) * wscale)
    X = rng.standard_normal((tokens, n))
    if outliers:
        X[:, rng.choice(n, max(1, n // 64), replace=False)] *= 20
    X = f32(X)
    return W, X


def _run(W, X, bits=4, G=32, B=64, damp=0.01, desc_act=False):
    S = oracle.hessian_S([X])
    P = oracle.prepare(S, damp, desc_act)
    r = oracle.gptq_quantize(W, P.U, bits, G, B, P.perm, P.dead)
    return P, r


def test_block_size_invariance():
    """Lazy batching only reorders the same updates: B in {G, 2G, n} agree."""
    W, X = _layer(48, 256, 1024, seed=1)
    S = oracle.hessian_S([X])
    P = oracle.prepare(S, 0.01, False)
    ref = oracle.gptq_quantize(W, P.U, 4, 32, 32)
    for B in (64, 256):
        r = oracle.gptq_quantize(W, P.U, 4, 32, B)
        assert np.array_equal(r.codes, ref.codes)
        assert np.allclose(r.scales, ref.scales, rtol=1e-12, atol=0)
        assert np.array_equal(r.zeros, ref.zeros)


def test_cholesky_route_equals_literal_obs_route():
    W, X = _layer(64, 192, 800, seed=2)
    S = oracle.hessian_S([X])
    for desc in (False, True):
        P = oracle.prepare(S, 0.01, desc)
        r = oracle.gptq_quantize(W, P.U, 3, 64, 64, P.perm, P.dead)
        codes, scales, zeros = oracle.gptq_obs_literal(W, P.Hd, 3, 64, P.perm)
        assert np.array_equal(codes, r.codes)
        assert np.allclose(scales, r.scales, rtol=1e-12, atol=0)
        assert np.array_equal(zeros, r.zeros)


def test_error_identity_W_minus_Q_equals_E_U():
    """delta = W - dequant(Q) = E U (processing order), hence sum e^2 = delta^T H_d delta."""
    W, X = _layer(40, 160, 640, seed=3)
    P, r = _run(W, X, bits=4, G=32, B=64)
    Wq = oracle.dequant_layer(r.codes, r.scales, r.zeros, r.g_idx)
    D = (W - Wq)[:, r.perm]
    assert np.abs(D - r.E @ P.U).max() < 1e-12
    lhs = np.sum(r.E ** 2, axis=1)
    rhs = np.einsum("rc,cd,rd->r", D, P.Hd, D)
    assert np.allclose(lhs, rhs, rtol=1e-9, atol=0)


def test_inverse_free_route_gives_the_same_codes():
    """A third route to the loop's decisions, needing no inverse of H_d: with R the upper
    factor of H_d = R R^T (a Cholesky factorization taken from the last index backwards),
    U = R^-1, so W - Q = E U gives E = (W - Q) R and the pre-rounding value of column j is
    w_j + sum_{k<j} d_k R_kj / R_jj with d_k = w_k - dequant(q_k) of the ORIGINAL weights.
    A group's parameters come from its columns' values when its first column j0 is reached
    (every column before j0 applied, none after); with T = D[:, :j0] R[:j0, group] and
    R U = I those values are W[:, group] + T inv(R[group, group]), so only the groups'
    diagonal blocks are inverted.  Written here column by column from R (no E, no lazy
    blocks, no U), it must give the oracle's codes, scales and zero-points (plain fp64
    decisions on both sides)."""
    from oracle.quantizer import group_params, quantize_codes
    W, X = _layer(32, 192, 800, seed=7)
    S = oracle.hessian_S([X])
    m, n = W.shape
    G = 64
    for desc in (False, True):
        P = oracle.prepare(S, 0.01, desc)
        assert not P.dead.any()
        r = oracle.gptq_quantize(W, P.U, 4, G, 64, P.perm, P.dead, exact=True)
        rev = np.arange(n)[::-1]
        R = np.linalg.cholesky(P.Hd[np.ix_(rev, rev)])[np.ix_(rev, rev)]
        assert np.allclose(R, np.triu(R), rtol=0, atol=0)
        Wp = W[:, P.perm].astype(np.float64)
        D = np.zeros_like(Wp)
        codes = np.zeros_like(Wp)
        scales, zeros = [], []
        for j in range(n):
            if j % G == 0:
                T = D[:, :j] @ R[:j, j:j + G]
                pre = Wp[:, j:j + G] + T @ np.linalg.inv(R[j:j + G, j:j + G])
                sc, zp = group_params(pre, 4, False, True)
                scales.append(sc)
                zeros.append(zp)
            w = Wp[:, j] + (D[:, :j] @ R[:j, j]) / R[j, j]
            codes[:, j] = quantize_codes(w, sc, zp, 4, True)
            D[:, j] = Wp[:, j] - sc * (codes[:, j] - zp)
        assert np.array_equal(codes, r.codes[:, P.perm])
        assert np.allclose(np.stack(scales, 1), r.scales, rtol=1e-12, atol=0)
        assert np.array_equal(np.stack(zeros, 1), r.zeros)


def test_diagonal_hessian_reduces_to_rtn():
    rng = np.random.default_rng(4)
    W = f32(rng.standard_normal((32, 128)) * 0.02)
    S = np.diag(rng.uniform(0.5, 5.0, 128))
    P = oracle.prepare(S, 0.01, False)
    r = oracle.gptq_quantize(W, P.U, 4, 32, 64)
    codes, scales, zeros = oracle.rtn_minmax(W, 4, 32)
    assert np.array_equal(r.codes, codes)
    assert np.array_equal(r.scales, scales) and np.array_equal(r.zeros, zeros)


def test_single_column_layer_is_rtn():
    rng = np.random.default_rng(5)
    W = f32(rng.standard_normal((64, 1)) * 0.02)
    X = f32(rng.standard_normal((100, 1)))
    P = oracle.prepare(oracle.hessian_S([X]), 0.01, False)
    r = oracle.gptq_quantize(W, P.U, 4, 1, 1)
    codes, _, _ = oracle.rtn_minmax(W, 4, 1)
    assert np.array_equal(r.codes, codes)


def test_huge_damping_reduces_to_rtn():
    W, X = _layer(64, 128, 512, seed=6)
    P, r = _run(W, X, bits=4, G=32, B=64, damp=1e4)
    codes, _, _ = oracle.rtn_minmax(W, 4, 32)
    assert np.array_equal(r.codes, codes)


def test_power_of_two_scaling_invariance():
    """X -> 2X (H -> 4H) and W -> 2W: identical codes and zeros, doubled scales."""
    W, X = _layer(32, 128, 512, seed=7)
    _, r1 = _run(W, X, G=32, B=64)
    _, r2 = _run(2 * W, 2 * X, G=32, B=64)
    assert np.array_equal(r1.codes, r2.codes)
    assert np.array_equal(r1.zeros, r2.zeros)
    assert np.array_equal(2 * r1.scales, r2.scales)


def test_row_permutation_equivariance():
    W, X = _layer(24, 96, 400, seed=8)
    P, r = _run(W, X, G=32, B=32)
    pr = np.random.default_rng(0).permutation(24)
    r2 = oracle.gptq_quantize(W[pr], P.U, 4, 32, 32)
    assert np.array_equal(r2.codes, r.codes[pr])
    assert np.array_equal(r2.scales, r.scales[pr])


def test_desc_act_equals_explicit_permutation():
    W, X = _layer(32, 128, 512, seed=9)
    S = oracle.hessian_S([X])
    P = oracle.prepare(S, 0.01, True)
    r = oracle.gptq_quantize(W, P.U, 4, 32, 64, P.perm, P.dead)
    # permute inputs explicitly, run with desc_act off, unpermute the codes
    Sp = S[np.ix_(P.perm, P.perm)]
    P2 = oracle.prepare(Sp, 0.01, False)
    r2 = oracle.gptq_quantize(W[:, P.perm], P2.U, 4, 32, 64)
    back = np.empty_like(r2.codes)
    back[:, P.perm] = r2.codes
    assert np.array_equal(back, r.codes)
    assert np.array_equal(r.scales, r2.scales)
    # g_idx: the group of each original column is its processing position // G
    assert np.array_equal(r.g_idx[P.perm], np.arange(128) // 32)


def test_identity_permutation_is_desc_act_off():
    W, X = _layer(16, 64, 256, seed=10)
    S = oracle.hessian_S([X])
    P = oracle.prepare(S, 0.01, False)
    a = oracle.gptq_quantize(W, P.U, 4, 32, 32)
    b = oracle.gptq_quantize(W, P.U, 4, 32, 32, perm=np.arange(64))
    assert np.array_equal(a.codes, b.codes)


def test_dead_column_is_zeroed():
    W, X = _layer(16, 64, 256, seed=11)
    X[:, 5] = 0.0
    P, r = _run(W, X, G=32, B=32)
    assert P.dead[5]
    Wq = oracle.dequant_layer(r.codes, r.scales, r.zeros, r.g_idx)
    assert np.all(Wq[:, 5] == 0.0)


def test_recon_error_closed_form_equals_direct():
    wl = synth.get_workload("layer256")
    W = synth.weight(wl)
    X = synth.x_all(wl, "x")
    S = oracle.hessian_S([X])
    P = oracle.prepare(S, 0.01, False)
    r = oracle.gptq_quantize(W, P.U, 4, 128, 128)
    Wq = oracle.dequant_layer(r.codes, r.scales, r.zeros, r.g_idx)
    a = oracle.recon_error_from_H(W, Wq, 2.0 * S)
    b = oracle.recon_error_direct(W, Wq, X)
    assert a == pytest.approx(b, rel=1e-10)


def test_gptq_beats_rtn_on_the_256_layer():
    wl = synth.get_workload("layer256")
    W = synth.weight(wl)
    X = synth.x_all(wl, "x")
    S = oracle.hessian_S([X])
    P = oracle.prepare(S, 0.01, False)
    r = oracle.gptq_quantize(W, P.U, 4, 128, 128)
    c, s, z = oracle.rtn_minmax(W, 4, 128)
    e_g = oracle.recon_error_from_H(W, oracle.dequant_layer(r.codes, r.scales, r.zeros, r.g_idx), 2 * S)
    e_r = oracle.recon_error_from_H(W, oracle.dequant_layer(c, s, z, np.arange(256) // 128), 2 * S)
    assert e_g < e_r


def test_gptq_beats_rtn_in_aggregate_on_tiny_layers():
    tot_g = tot_r = 0.0
    for seed in range(40):
        W, X = _layer(8, 16, 64, seed=100 + seed, outliers=False)
        S = oracle.hessian_S([X])
        P = oracle.prepare(S, 0.01, False)
        r = oracle.gptq_quantize(W, P.U, 3, 8, 8)
        c, s, z = oracle.rtn_minmax(W, 3, 8)
        tot_g += oracle.recon_error_from_H(W, oracle.dequant_layer(r.codes, r.scales, r.zeros, r.g_idx), P.H)
        tot_r += oracle.recon_error_from_H(W, oracle.dequant_layer(c, s, z, np.arange(16) // 8), P.H)
    assert tot_g < tot_r


def _brute_force_best(w, scale, zero, maxq, H):
    n = w.shape[0]
    best = np.inf
    for combo in itertools.product(range(maxq + 1), repeat=n):
        d = w - (np.array(combo, dtype=np.float64) - zero) * scale
        best = min(best, float(d @ H @ d))
    return best


@pytest.mark.parametrize("bits,n", [(2, 5), (3, 4)])
def test_brute_force_optimum_bounds_gptq_and_rtn(bits, n):
    """One group per row (same grid for all three): OPT <= GPTQ and OPT <= RTN."""
    maxq = 2 ** bits - 1
    for seed in range(12):
        rng = np.random.default_rng(300 + seed)
        W = f32(rng.standard_normal((1, n)) * 0.02)
        X = rng.standard_normal((4 * n, n)) @ rng.standard_normal((n, n))
        S = oracle.hessian_S([X])
        P = oracle.prepare(S, 0.01, False)
        r = oracle.gptq_quantize(W, P.U, bits, n, n)
        c, s, z = oracle.rtn_minmax(W, bits, n)
        assert np.array_equal(r.scales, s) and np.array_equal(r.zeros, z)
        dg = W[0] - oracle.dequantize(r.codes[0], s[0, 0], z[0, 0])
        dr = W[0] - oracle.dequantize(c[0], s[0, 0], z[0, 0])
        eg, er = float(dg @ P.H @ dg), float(dr @ P.H @ dr)
        opt = _brute_force_best(W[0], s[0, 0], z[0, 0], maxq, P.H)
        assert opt <= eg * (1 + 1e-12) and opt <= er * (1 + 1e-12)


def test_two_columns_gptq_never_worse_than_rtn():
    """n = 2, one group: GPTQ rounds the first column like RTN and then picks the best
    second code given the first, so its error cannot exceed RTN's."""
    for seed in range(400):
        rng = np.random.default_rng(1000 + seed)
        W = f32(rng.standard_normal((1, 2)) * 0.05)
        A = rng.standard_normal((2, 2))
        S = A @ A.T + 1e-3 * np.eye(2)
        P = oracle.prepare(S, 0.01, False)
        r = oracle.gptq_quantize(W, P.U, 2, 2, 2)
        c, s, z = oracle.rtn_minmax(W, 2, 2)
        dg = W[0] - oracle.dequantize(r.codes[0], s[0, 0], z[0, 0])
        dr = W[0] - oracle.dequantize(c[0], s[0, 0], z[0, 0])
        assert dg @ P.H @ dg <= dr @ P.H @ dr * (1 + 1e-12) + 1e-300


def test_replay_accepts_own_result_and_flags_a_hard_mismatch():
    W, X = _layer(32, 128, 512, seed=12)
    P, r = _run(W, X, G=32, B=64)
    rep = oracle.replay_check(W, P.U, 4, 32, 64, P.perm, P.dead, r.codes_proc, r.scales, r.zeros)
    assert rep.mismatches == 0 and rep.hard == 0 and rep.scale_max_rel == 0.0
    bad = r.codes_proc.copy()
    bad[3, 17] = (bad[3, 17] + 2) % 16
    rep = oracle.replay_check(W, P.U, 4, 32, 64, P.perm, P.dead, bad, r.scales, r.zeros)
    assert rep.hard >= 1
    # row error of the replay equals sum of e^2 of the oracle itself
    rep = oracle.replay_check(W, P.U, 4, 32, 64, P.perm, P.dead, r.codes_proc, r.scales, r.zeros)
    assert np.allclose(rep.row_err, np.sum(r.E ** 2, axis=1), rtol=1e-12)


def test_group_size_minus_one_is_one_group_per_row():
    W, X = _layer(16, 64, 256, seed=13)
    S = oracle.hessian_S([X])
    P = oracle.prepare(S, 1e4, False)
    r = oracle.gptq_quantize(W, P.U, 4, -1, 32)
    c, s, z = oracle.rtn_minmax(W, 4, -1)
    assert r.scales.shape == (16, 1)
    assert np.array_equal(r.codes, c)
