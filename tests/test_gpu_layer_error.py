"""GPU parity: gptq_layer_error, the layer's output error delta_r S delta_r^T per row.

The layer objective ("LLM quantization principles" section 3.1) of a quantized
layer, from its original-order codes, scales, zeros and g_idx and the raw
calibration second moments S.  Checked per row against the oracle's quadratic
form through H = 2S (recon_error_from_H, fp64), within a bound on the device's
fp32 rounding, and summed over rows against the oracle's token-by-token
||W X^T - W_q X^T||^2 (recon_error_direct, which never forms S).
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.quantizer import f32

from gpu_util import dev, host, need_gpu, say, storage_dtype, torch

pytestmark = pytest.mark.gpu

EPS32 = 2.0 ** -24

CASES = [
    # name, m, n, tokens, bits, G, desc_act, w dtype, quantizer
    ("gptq_g128", 96, 512, 2048, 4, 128, False, "bf16", "gptq"),
    ("gptq_desc_g64", 80, 640, 2048, 4, 64, True, "bf16", "gptq"),
    ("gptq_row_group_f32", 64, 384, 1024, 3, -1, False, "f32", "gptq"),
    ("rtn_g32_ragged", 77, 333, 1000, 4, 32, False, "f32", "rtn"),
]


def _inputs(name, m, n, tokens, bits, G, desc, wdt, kind, seed):
    wl = synth.custom_workload(name, m, n, tokens, tokens, w_sigma=0.02, w_dtype=wdt,
                               x_dist="normal", outlier_frac=0.02, outlier_mult=20.0,
                               bits=bits, group_size=G, desc_act=desc, workload_id=600 + seed)
    W = synth.weight(wl)
    X = synth.x_all(wl, "x")
    S = f32(oracle.hessian_S([X]))
    if kind == "gptq":
        P = oracle.prepare(S, float(np.float32(0.01)), desc)
        r = oracle.gptq_quantize(W, P.U, bits, G, 128, P.perm, P.dead)
        codes, scales, zeros, g_idx = r.codes, r.scales, r.zeros, r.g_idx
    else:
        codes, scales, zeros = oracle.rtn_minmax(W, bits, G)
        g_idx = np.arange(n) // (G if G > 0 else n)
    return W, X, S, codes, scales, zeros, np.asarray(g_idx)


def _run(W, S, codes, scales, zeros, g_idx, wdt):
    q = need_gpu()
    m, n = W.shape
    err = torch.empty(m, dtype=torch.float64, device="cuda")
    q.gptq_layer_error(dev(W, storage_dtype(wdt)), dev(codes.astype(np.uint8), torch.uint8),
                       dev(f32(scales), torch.float32), dev(f32(zeros), torch.float32),
                       dev(g_idx.astype(np.int32), torch.int32), dev(S, torch.float32), err)
    torch.cuda.synchronize()
    return host(err)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_error_matches_oracle(case):
    name, m, n, tokens, bits, G, desc, wdt, kind = case
    W, X, S, codes, scales, zeros, g_idx = _inputs(*case, seed=CASES.index(case))
    say("layer error", name, m, n)
    err = _run(W, S, codes, scales, zeros, g_idx, wdt)
    Wq = oracle.dequant_layer(codes, scales, zeros, g_idx)
    H = 2.0 * np.asarray(S, np.float64)
    ref = np.array([oracle.recon_error_from_H(W[r:r + 1], Wq[r:r + 1], H) for r in range(m)])
    # fp32 differences (two roundings, relative to |w| + |w_q|) and an fp32
    # product with n-term sums: every rounding is within n + 8 units of 2^-24
    # of the quadratic form of the magnitudes
    A = np.abs(W).astype(np.float64) + np.abs(Wq)
    bound = 4.0 * (n + 8) * EPS32 * np.sum((A @ np.abs(np.asarray(S, np.float64))) * A, axis=1)
    dev_ = np.abs(err - ref)
    print(f"{name}: max |err - ref| / bound {float((dev_ / bound).max()):.3e}, "
          f"median relative {float(np.median(dev_ / ref)):.2e}")
    assert np.all(dev_ <= bound)
    assert float(np.median(dev_ / ref)) <= 1e-5
    # the sum over rows is the layer objective, taken over the tokens directly
    direct = oracle.recon_error_direct(W, Wq, X)
    assert abs(float(err.sum()) - direct) <= float(bound.sum()) + 1e-9 * direct


def test_layer_error_is_zero_for_exact_weights_and_deterministic():
    """Weights on the quantization grid give zero error; two calls agree bit for bit."""
    q = need_gpu()
    m, n, tokens = 64, 256, 512
    W, X, S, codes, scales, zeros, g_idx = _inputs("exact", m, n, tokens, 4, 64, False, "f32",
                                                   "rtn", seed=9)
    Wq = f32(oracle.dequant_layer(codes, scales, zeros, g_idx))
    e0 = _run(Wq, S, codes, scales, zeros, g_idx, "f32")
    assert np.all(e0 == 0.0)
    e1 = _run(W, S, codes, scales, zeros, g_idx, "f32")
    e2 = _run(W, S, codes, scales, zeros, g_idx, "f32")
    assert np.array_equal(e1, e2) and np.all(e1 > 0.0)
