"""GPU parity: gptq_quantize_layer (column loop) against the oracle, given the oracle's U.

Feeding both sides the same U (the oracle's, rounded to fp32) isolates the
block column-quantize and trailing-update kernels from the Hessian and
prepare stages.  Bars: codes identical on >= 99.9 % of entries free-running;
replay (the oracle's loop following the device's choices, either neighbour
accepted within 1e-3 step of a rounding tie) finds no hard mismatch; scales
within 1e-4 relative in replay; reconstruction error within 1e-3 relative.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.quantizer import f32

from gpu_util import dev, host, match_rate, need_gpu, root_cascade, say, storage_dtype, torch

pytestmark = pytest.mark.gpu

QCASES = [
    # m, n, tokens, G, bits, desc_act, wdt, xdist
    (64, 256, 1024, 128, 4, False, "bf16", "normal"),
    (40, 384, 2048, 64, 3, True, "bf16", "student_t4"),
    (33, 200, 1024, 32, 4, False, "f32", "normal"),      # ragged: last block of 72 columns
    (16, 130, 512, 8, 2, False, "bf16", "laplace"),      # last block of 2 columns
    (20, 256, 1024, -1, 4, False, "bf16", "normal"),     # one group per row
    (24, 512, 2048, 16, 4, True, "bf16", "laplace"),
    (300, 640, 4096, 128, 4, False, "bf16", "normal"),   # rows span several tiles
    (17, 64, 256, 64, 8, False, "f32", "normal"),        # n < one block
]


def run_case(q, m, n, tokens, G, bits, desc, wdt, xdist, sym=False, dead_cols=(),
             static=False):
    wl = synth.custom_workload("qc", m, n, tokens, min(tokens, 2048), w_dtype=wdt, x_dist=xdist,
                               outlier_frac=0.01, outlier_mult=20.0, bits=bits, group_size=G,
                               desc_act=desc, sym=sym, workload_id=300 + m + n)
    W = synth.weight(wl)
    X = synth.x_all(wl, "x")
    if dead_cols:
        X[:, list(dead_cols)] = 0.0
    S = oracle.hessian_S([X])
    P = oracle.prepare(S, float(np.float32(0.01)), desc)
    U32 = f32(P.U)  # both sides get the same fp32 U
    ref = oracle.gptq_quantize(W, U32, bits, G, 128, P.perm, P.dead, sym, static_groups=static)
    cfg = q.make_config(bits, G, desc_act=desc, sym=sym, static_groups=static)
    ng = ref.scales.shape[1]
    codes = torch.empty((m, n), dtype=torch.uint8, device="cuda")
    scales = torch.empty((m, ng), dtype=torch.float32, device="cuda")
    zeros = torch.empty((m, ng), dtype=torch.float32, device="cuda")
    g_idx = torch.empty(n, dtype=torch.int32, device="cuda")
    row_err = torch.empty(m, dtype=torch.float32, device="cuda")
    info = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    say("quantize", m, n, G, bits, desc, wdt, xdist, sym, static)
    q.gptq_quantize_layer(dev(W, storage_dtype(wdt)), dev(U32.astype(np.float32), torch.float32),
                          cfg, codes, scales, zeros, perm=dev(P.perm.astype(np.int32), torch.int32),
                          dead=dev(P.dead.astype(np.uint8), torch.uint8), g_idx=g_idx,
                          row_err=row_err, info=info)
    torch.cuda.synchronize()
    return W, X, S, P, U32, ref, host(codes), host(scales), host(zeros), host(g_idx), \
        host(row_err), int(host(info)[0])


@pytest.mark.parametrize("m,n,tokens,G,bits,desc,wdt,xdist", QCASES)
def test_quantize_given_oracle_U(m, n, tokens, G, bits, desc, wdt, xdist):
    q = need_gpu()
    W, X, S, P, U32, ref, codes, scales, zeros, g_idx, row_err, info = run_case(
        q, m, n, tokens, G, bits, desc, wdt, xdist)
    assert info == 0
    assert np.array_equal(g_idx, ref.g_idx)
    rate = match_rate(codes, ref.codes)
    roots, casc = root_cascade(codes, ref.codes, P.perm)
    print(f"match {rate:.6f} roots {roots} cascaded {casc}")
    assert rate >= 0.999
    codes_proc = codes.astype(np.float64)[:, P.perm]
    rep = oracle.replay_check(W, U32, bits, G, 128, P.perm, P.dead, codes_proc, scales, zeros)
    print(f"replay: mism {rep.mismatches} ties {rep.ties} hard {rep.hard} "
          f"zero-hard {rep.zero_hard} scale rel {rep.scale_max_rel:.2e}")
    assert rep.hard == 0 and rep.zero_hard == 0
    assert rep.scale_max_rel <= 1e-4
    # row error sum e^2 against the replay (same trajectory)
    assert np.allclose(row_err, rep.row_err, rtol=1e-3, atol=1e-12 * rep.row_err.max())
    # layer reconstruction error ||WX - QX||^2 from the device's codes
    Wq = oracle.dequant_layer(codes.astype(np.float64), scales.astype(np.float64),
                              zeros.astype(np.float64), g_idx)
    Wq_ref = oracle.dequant_layer(ref.codes, ref.scales, ref.zeros, ref.g_idx)
    H = 2.0 * S
    e_dev = oracle.recon_error_from_H(W, Wq, H)
    e_ref = oracle.recon_error_from_H(W, Wq_ref, H)
    assert abs(e_dev - e_ref) <= 1e-3 * e_ref


@pytest.mark.parametrize("bits,desc", [(4, False), (3, True)])
def test_quantize_symmetric_and_dead_columns(bits, desc):
    q = need_gpu()
    W, X, S, P, U32, ref, codes, scales, zeros, g_idx, row_err, info = run_case(
        q, 32, 256, 1024, 64, bits, desc, "bf16", "normal", sym=True, dead_cols=(3, 200))
    assert info == 0
    assert P.dead[3] and P.dead[200]
    assert match_rate(codes, ref.codes) >= 0.999
    Wq = oracle.dequant_layer(codes.astype(np.float64), scales.astype(np.float64),
                              zeros.astype(np.float64), g_idx)
    assert np.all(Wq[:, [3, 200]] == 0.0)
    assert np.all(zeros == float(2 ** (bits - 1)))
    # the symmetric loop replayed on the oracle's arithmetic, following the device's choices
    codes_proc = codes.astype(np.float64)[:, P.perm]
    rep = oracle.replay_check(W, U32, bits, 64, 128, P.perm, P.dead, codes_proc, scales, zeros,
                              sym=True)
    print(f"replay (sym): mism {rep.mismatches} ties {rep.ties} hard {rep.hard} "
          f"zero-hard {rep.zero_hard} scale rel {rep.scale_max_rel:.2e}")
    assert rep.hard == 0 and rep.zero_hard == 0
    assert rep.scale_max_rel <= 1e-4
    assert np.allclose(row_err, rep.row_err, rtol=1e-3, atol=1e-12 * rep.row_err.max())


def test_quantize_reports_non_finite_weights():
    q = need_gpu()
    m, n = 16, 128
    W = np.zeros((m, n), dtype=np.float32)
    W[3, 7] = np.inf
    U = np.eye(n, dtype=np.float32)
    cfg = q.make_config(4, 128)
    codes = torch.empty((m, n), dtype=torch.uint8, device="cuda")
    scales = torch.empty((m, 1), dtype=torch.float32, device="cuda")
    zeros = torch.empty((m, 1), dtype=torch.float32, device="cuda")
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("quantize non-finite")
    q.gptq_quantize_layer(dev(W, torch.float32), dev(U, torch.float32), cfg, codes, scales, zeros,
                          info=info)
    torch.cuda.synchronize()
    assert int(host(info)[0]) == -1


def test_quantize_deterministic():
    q = need_gpu()
    outs = [run_case(q, 96, 384, 1024, 128, 4, True, "bf16", "normal")[6] for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


VCASES = [
    # m, n, tokens, G, bits, desc_act, static, dead columns
    (64, 256, 1024, 128, 4, True, True, ()),       # static groups with desc_act
    (40, 384, 2048, 64, 3, True, True, (5, 200)),  # static, dead columns
    (33, 200, 1024, 32, 4, False, True, ()),       # static, ragged last block
    (16, 640, 1024, 256, 4, True, True, ()),       # static groups larger than a block
    (24, 1024, 2048, 256, 4, True, False, ()),     # a group spanning two blocks
    (20, 1280, 2048, 512, 3, False, False, ()),    # four blocks; last group cut at n
    (12, 2304, 2048, 256, 4, True, False, (7,)),   # groups across a super-block boundary
]


@pytest.mark.parametrize("m,n,tokens,G,bits,desc,static,dead", VCASES)
def test_quantize_grouping_variants(m, n, tokens, G, bits, desc, static, dead):
    q = need_gpu()
    W, X, S, P, U32, ref, codes, scales, zeros, g_idx, row_err, info = run_case(
        q, m, n, tokens, G, bits, desc, "bf16", "student_t4", dead_cols=dead, static=static)
    assert info == 0
    assert np.array_equal(g_idx, ref.g_idx)
    if static:
        _, s_rtn, z_rtn = oracle.rtn_minmax(np.where(P.dead[None, :], 0.0, W), bits, G)
        assert np.array_equal(scales.astype(np.float64), s_rtn)
        assert np.array_equal(zeros.astype(np.float64), z_rtn)
    rate = match_rate(codes, ref.codes)
    print(f"match {rate:.6f}")
    assert rate >= 0.999
    rep = oracle.replay_check(W, U32, bits, G, 128, P.perm, P.dead,
                              codes.astype(np.float64)[:, P.perm], scales, zeros,
                              static_groups=static)
    print(f"replay: mism {rep.mismatches} ties {rep.ties} hard {rep.hard} "
          f"zero-hard {rep.zero_hard} scale rel {rep.scale_max_rel:.2e}")
    assert rep.hard == 0 and rep.zero_hard == 0
    assert rep.scale_max_rel <= 1e-4
