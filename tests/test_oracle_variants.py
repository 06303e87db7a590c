"""Pins for the grouping variants of the oracle's column loop (CPU only).

Static groups: a variant of the loop of "GPTQ deep dive" §3.1 step 3 in which
each group's scale and zero-point are computed once, from the original
weights, for groups of consecutive original columns (the pages do not describe
it; this is the plain reading of the name, and with desc_act it keeps g_idx =
c // G).  Groups larger than the 128-column block: group_size a multiple of
block_size gives what block_size = group_size gives ("AWQ, MinMax, GPTQ
calibration in Model Optimizer" §4 asks for block_size to be a multiple of
group_size; the "Calibration algorithms guide" sweeps group sizes up to 512).
Pinned by the RTN limit (no compensation with a diagonal U), by the
parameters' closed form (they are RTN's), by g_idx, by blocking invariance and
by the replay of the oracle's own result.
"""
import numpy as np
import pytest

import oracle
import synth


def _layer(m, n, tokens, seed):
    wl = synth.custom_workload("v", m, n, tokens, tokens, w_dtype="f32", x_dtype="f32",
                               workload_id=300 + seed)
    return synth.weight(wl).astype(np.float64), synth.x_all(wl, "x").astype(np.float64)


@pytest.mark.parametrize("bits,G", [(4, 32), (3, 64), (2, 16)])
def test_static_group_params_are_rtn_params(bits, G):
    W, X = _layer(24, 192, 512, 1)
    P = oracle.prepare(oracle.hessian_S([X]), 0.01, True)
    r = oracle.gptq_quantize(W, P.U, bits, G, 64, P.perm, P.dead, static_groups=True)
    _, s_rtn, z_rtn = oracle.rtn_minmax(W, bits, G)
    assert np.array_equal(r.scales, s_rtn) and np.array_equal(r.zeros, z_rtn)
    assert np.array_equal(r.g_idx, np.arange(192) // G)


def test_static_groups_without_compensation_are_rtn():
    """A diagonal U pushes no error onto other columns: every column is rounded
    with its ORIGINAL group's parameters, whatever the processing order."""
    rng = np.random.default_rng(2)
    m, n, G = 16, 128, 32
    W = rng.standard_normal((m, n)) * 0.02
    U = np.diag(rng.uniform(0.5, 2.0, n))
    perm = rng.permutation(n)
    r = oracle.gptq_quantize(W, U, 4, G, 32, perm, None, static_groups=True)
    codes, _, _ = oracle.rtn_minmax(W, 4, G)
    assert np.array_equal(r.codes, codes)
    # the dynamic grouping of the same permuted order is a different quantization
    d = oracle.gptq_quantize(W, U, 4, G, 32, perm, None)
    assert not np.array_equal(d.codes, codes)


def test_static_groups_replay_and_beat_rtn_in_aggregate():
    W, X = _layer(32, 256, 1024, 3)
    S = oracle.hessian_S([X])
    H = 2.0 * S
    P = oracle.prepare(S, 0.01, True)
    r = oracle.gptq_quantize(W, P.U, 3, 64, 128, P.perm, P.dead, static_groups=True)
    rep = oracle.replay_check(W, P.U, 3, 64, 128, P.perm, P.dead, r.codes_proc, r.scales,
                              r.zeros, static_groups=True)
    assert rep.mismatches == 0 and rep.zero_mismatches == 0 and rep.scale_max_rel == 0.0
    codes, s, z = oracle.rtn_minmax(W, 3, 64)
    e_gptq = oracle.recon_error_from_H(W, oracle.dequant_layer(r.codes, r.scales, r.zeros,
                                                               r.g_idx), H)
    e_rtn = oracle.recon_error_from_H(W, oracle.dequant_layer(codes, s, z,
                                                              np.arange(256) // 64), H)
    assert e_gptq < e_rtn


@pytest.mark.parametrize("G", [256, 512])
def test_group_larger_than_block_equals_block_of_group_size(G):
    W, X = _layer(16, 1024, 2048, 4)
    P = oracle.prepare(oracle.hessian_S([X]), 0.01, True)
    a = oracle.gptq_quantize(W, P.U, 4, G, 128, P.perm, P.dead)
    b = oracle.gptq_quantize(W, P.U, 4, G, G, P.perm, P.dead)
    assert np.array_equal(a.codes, b.codes)
    assert np.allclose(a.scales, b.scales, rtol=1e-12, atol=0)
    assert np.array_equal(a.zeros, b.zeros)
    g = np.empty(1024, dtype=np.int64)
    g[P.perm] = np.arange(1024) // G
    assert np.array_equal(a.g_idx, g)
    rep = oracle.replay_check(W, P.U, 4, G, 128, P.perm, P.dead, a.codes_proc, a.scales,
                              a.zeros)
    assert rep.mismatches == 0 and rep.scale_max_rel == 0.0


def test_group_larger_than_block_without_compensation_is_rtn():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((8, 512)) * 0.02
    U = np.diag(rng.uniform(0.5, 2.0, 512))
    r = oracle.gptq_quantize(W, U, 4, 256, 128)
    codes, scales, zeros = oracle.rtn_minmax(W, 4, 256)
    assert np.array_equal(r.codes, codes) and np.array_equal(r.scales, scales)
