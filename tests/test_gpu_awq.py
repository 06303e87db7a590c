"""GPU parity: AWQ-lite scale search and awq_clip against the oracle.

The activation statistics are checked against the oracle's fp64 sums.  The alpha
search is checked on what must agree.  The device computes s with powf and the
oracle in fp64, so W' = W diag(s) can differ in its last bit, and a value of W'
that sits on a rounding tie (with symmetric parameters the group's most negative
value always does: it maps to -(2^(b-1) - 1/2) steps) may take either code.
Every candidate's output error must lie within 1e-3 of the oracle's plus the
most that those tie decisions can move it (|dL| <= 2 |e| |S D^T| + |e| |S| |e|^T
per row, e the possible changes); the chosen alpha must be the smallest error
for some resolution of the ties, and s within 1e-5.
The clip search is checked given the device's s (so that both sides quantize
the same W'): the chosen clip's error within 1e-4 of the group's smallest, and
the codes, scales and zero-points bit-identical to the oracle's quantizer at the
device's chosen clips.  AWQ must beat plain group min-max on a layer with
outlier activation channels.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import awq

from gpu_util import dev, host, need_gpu, say, torch

pytestmark = pytest.mark.gpu

EPS32 = 2.0 ** -24


def _lite_reference(W, S, xm, bits, G, sym):
    """Per candidate alpha: the oracle's output error and the bound on how far
    rounding-tie decisions (values of W' within 2^-20 relative of a half step, a
    few units in the last place of s and of the division, whose two candidate
    codes differ after clamping) can move it."""
    from oracle.quantizer import group_params
    n = W.shape[1]
    maxq = 2 ** bits - 1
    w_mean = awq.weight_absmean(W)
    losses, bounds = [], []
    for a in awq.ALPHAS:
        s = awq.awq_scales(xm, w_mean, a)
        Ws = W * s
        q, sc, z = awq.quantize_groups(Ws, bits, G, sym)
        D = awq.dequant_groups(q, sc, z, G) / s - W
        E = np.zeros_like(W)
        for k, g0 in enumerate(range(0, n, G)):
            g1 = min(n, g0 + G)
            scale, zero = group_params(Ws[:, g0:g1], bits, sym)
            pre = oracle.f32(oracle.f32(Ws[:, g0:g1]) / scale[:, None])
            lo = np.floor(pre)
            near = np.abs(pre - lo - 0.5) < 2.0 ** -20 * np.maximum(np.abs(pre), 1.0)
            qlo = np.clip(lo + zero[:, None], 0, maxq)
            qhi = np.clip(lo + 1 + zero[:, None], 0, maxq)
            E[:, g0:g1] = np.where(near, np.abs(qhi - qlo) * scale[:, None], 0.0) / s[g0:g1]
        losses.append(awq.output_error(D, S))
        bounds.append(float(np.sum(2 * E * np.abs(D @ S)) + np.sum((E @ np.abs(S)) * E)))
    return np.array(losses), np.array(bounds)


def _check_lite(losses_dev, alpha_dev, W, S, xm, bits, G, sym, s_dev):
    L, B = _lite_reference(W, S, xm, bits, G, sym)
    k = int(round(alpha_dev * 10))
    dev_l = np.asarray(losses_dev, np.float64)
    rel = np.abs(dev_l - L) / L
    print(f"  alpha device {alpha_dev:.2f} oracle {awq.ALPHAS[int(np.argmin(L))]:.2f}; loss rel "
          f"diff max {rel.max():.2e}, tie bound max {float((B / L).max()):.2e}", flush=True)
    assert abs(alpha_dev - 0.1 * k) < 1e-6
    assert np.all(np.abs(dev_l - L) <= 1e-3 * L + B)
    assert L[k] - B[k] <= float(np.min(L + B)) * (1 + 1e-3)
    s_ref = awq.awq_scales(xm, awq.weight_absmean(W), 0.1 * k)
    # at the device's own s (the same fp32 W', so the same tie decisions) the
    # chosen candidate's error matches without the tie allowance
    q, sc, z = awq.quantize_groups(W * s_dev, bits, G, sym)
    L_own = awq.output_error(awq.dequant_groups(q, sc, z, G) / s_dev - W, S)
    assert abs(dev_l[k] - L_own) <= 1e-3 * L_own, (dev_l[k], L_own)
    return k, s_ref


def _run(q, W, X, bits, G, sym=False):
    m, n = W.shape
    Wd = dev(W.astype(np.float32), torch.bfloat16)
    Xd = dev(X.astype(np.float32), torch.bfloat16)
    S = torch.zeros((n, n), dtype=torch.float32, device="cuda")
    q.gptq_hessian_accumulate(S, Xd)
    absum = torch.zeros(n, dtype=torch.float32, device="cuda")
    q.awq_activation_absum(Xd, absum)
    s = torch.empty(n, dtype=torch.float32, device="cuda")
    alpha = torch.empty(1, dtype=torch.float32, device="cuda")
    losses = torch.empty(11, dtype=torch.float32, device="cuda")
    q.awq_lite(Wd, S, absum, X.shape[0], bits, G, s, alpha, losses, sym=sym)
    ng = -(-n // G)
    codes = torch.empty((m, n), dtype=torch.uint8, device="cuda")
    scales = torch.empty((m, ng), dtype=torch.float32, device="cuda")
    zeros = torch.empty((m, ng), dtype=torch.float32, device="cuda")
    cidx = torch.empty((m, ng), dtype=torch.uint8, device="cuda")
    q.awq_clip_quantize(Wd, S, s, bits, G, codes, scales, zeros, cidx, sym=sym)
    torch.cuda.synchronize()
    S_dev = host(S).astype(np.float64)
    S_full = np.tril(S_dev) + np.tril(S_dev, -1).T
    return dict(S=S_full, absum=host(absum).astype(np.float64), s=host(s).astype(np.float64),
                alpha=float(host(alpha)[0]), losses=host(losses).astype(np.float64),
                codes=host(codes).astype(np.int64), scales=host(scales).astype(np.float64),
                zeros=host(zeros).astype(np.float64), cidx=host(cidx).astype(np.int64))


def _check(r, W, X, bits, G, sym=False):
    tokens, n = X.shape
    absum_ref = np.abs(X).sum(axis=0)
    # fp64 sums on the device, rounded once to fp32
    assert np.all(np.abs(r["absum"] - absum_ref) <= EPS32 * absum_ref * 1.0001)
    xm = r["absum"] / tokens
    S = r["S"]  # the device Hessian (its parity is tested on its own)
    _, s_ref = _check_lite(r["losses"], r["alpha"], W, S, xm, bits, G, sym, r["s"])
    assert np.all(np.abs(r["s"] - s_ref) <= 1e-5 * s_ref)
    # the clip search on the device's W' = W diag(s)
    clip = awq.awq_clip(W, S, r["s"], bits, G, sym)
    errs = clip.errors
    chosen = np.take_along_axis(errs, r["cidx"][:, :, None], axis=2)[:, :, 0]
    best = errs.min(axis=2)
    scale_err = np.abs(errs).max(axis=2)
    assert np.all(chosen <= best + 1e-4 * scale_err + 1e-30)
    agree = float(np.mean(r["cidx"] == clip.ratio_idx))
    ratios = awq.CLIP_RATIOS[r["cidx"]]
    Ws = oracle.f32(W * r["s"])
    amax = np.stack([np.abs(Ws[:, g0:g0 + G]).max(axis=1) for g0 in range(0, n, G)], axis=1)
    codes, scales, zeros = awq.quantize_groups(Ws, bits, G, sym,
                                               ranges=oracle.f32(amax * oracle.f32(ratios)))
    print(f"  clip choices equal to the oracle's {agree:.4f}", flush=True)
    assert np.array_equal(r["codes"], codes)
    assert np.array_equal(r["scales"], scales) and np.array_equal(r["zeros"], zeros)


CASES = [
    # m, n, tokens, bits, G, sym, outliers
    (64, 256, 2048, 4, 128, False, 4),
    (96, 512, 4096, 3, 64, False, 8),
    (40, 384, 1024, 4, 32, True, 3),
    (33, 200, 1000, 4, 40, False, 2),   # odd sizes
    (17, 150, 500, 4, 64, False, 2),    # ragged last group, n not a multiple of 4
]


@pytest.mark.parametrize("m,n,tokens,bits,G,sym,nout", CASES)
def test_awq_against_oracle(m, n, tokens, bits, G, sym, nout):
    q = need_gpu()
    rng = np.random.default_rng(m + n + bits)
    W = synth.round_to_bf16((rng.standard_normal((m, n)) * 0.02).astype(np.float32)).astype(np.float64)
    X = rng.standard_normal((tokens, n))
    X[:, rng.choice(n, nout, replace=False)] *= 30.0
    X = synth.round_to_bf16(X.astype(np.float32)).astype(np.float64)
    say("awq", m, n, tokens, bits, G, sym)
    r = _run(q, W, X, bits, G, sym)
    _check(r, W, X, bits, G, sym)


def test_awq_beats_plain_minmax_on_outlier_channels():
    q = need_gpu()
    rng = np.random.default_rng(9)
    m, n, tokens, bits, G = 128, 512, 4096, 3, 128
    W = synth.round_to_bf16((rng.standard_normal((m, n)) * 0.02).astype(np.float32)).astype(np.float64)
    X = rng.standard_normal((tokens, n))
    X[:, rng.choice(n, 6, replace=False)] *= 40.0
    X = synth.round_to_bf16(X.astype(np.float32)).astype(np.float64)
    say("awq vs rtn", m, n)
    r = _run(q, W, X, bits, G)
    S = r["S"]
    W_awq = awq.dequant_groups(r["codes"], r["scales"], r["zeros"], G) / r["s"]
    c, sc, z = oracle.rtn_minmax(W, bits, G)
    W_rtn = oracle.dequant_layer(c, sc, z, np.arange(n) // G)
    e_awq = awq.output_error(W_awq - W, S)
    e_rtn = awq.output_error(W_rtn - W, S)
    print(f"  output error: AWQ {e_awq:.4e}, min-max {e_rtn:.4e}", flush=True)
    assert r["alpha"] > 0 and e_awq < 0.8 * e_rtn


@pytest.mark.timeout(900)
def test_awq_full_size_llama7b_attention():
    """The Llama-7B attention projection workload (4096 x 4096, 262144 tokens,
    4-bit g128): every candidate's error, the chosen alpha and s, and the clip
    search and codes on 32 sampled rows."""
    q = need_gpu()
    wl = synth.get_workload("llama7b_attn")
    ls = wl.layer()
    xs = wl.xs[ls.x]
    n, N = ls.n, xs.tokens
    W = synth.weight(wl, ls.name).astype(np.float64)
    Xd = torch.empty((N, n), dtype=torch.bfloat16, device="cuda")
    absum_ref = np.zeros(n)
    for c0 in range(0, xs.chunks, 16):
        idx = list(range(c0, min(xs.chunks, c0 + 16)))
        Xh = synth.x_all(wl, ls.x, chunks=idx)
        Xd[c0 * xs.chunk_len:(c0 + len(idx)) * xs.chunk_len].copy_(torch.from_numpy(Xh).to(torch.bfloat16))
        absum_ref += np.abs(Xh.astype(np.float64)).sum(axis=0)
    say("awq full size", ls.m, n, N)
    Wd = dev(W.astype(np.float32), torch.bfloat16)
    S = torch.zeros((n, n), dtype=torch.float32, device="cuda")
    q.gptq_hessian_accumulate(S, Xd)
    absum = torch.zeros(n, dtype=torch.float32, device="cuda")
    q.awq_activation_absum(Xd, absum)
    s = torch.empty(n, dtype=torch.float32, device="cuda")
    alpha = torch.empty(1, dtype=torch.float32, device="cuda")
    losses = torch.empty(11, dtype=torch.float32, device="cuda")
    q.awq_lite(Wd, S, absum, N, 4, 128, s, alpha, losses)
    codes = torch.empty((ls.m, n), dtype=torch.uint8, device="cuda")
    scales = torch.empty((ls.m, n // 128), dtype=torch.float32, device="cuda")
    zeros = torch.empty((ls.m, n // 128), dtype=torch.float32, device="cuda")
    cidx = torch.empty((ls.m, n // 128), dtype=torch.uint8, device="cuda")
    q.awq_clip_quantize(Wd, S, s, 4, 128, codes, scales, zeros, cidx)
    torch.cuda.synchronize()
    absum_d = host(absum).astype(np.float64)
    assert np.all(np.abs(absum_d - absum_ref) <= EPS32 * absum_ref * 1.0001)
    S_dev = host(S).astype(np.float64)
    S_full = np.tril(S_dev) + np.tril(S_dev, -1).T
    del Xd, S
    xm = absum_d / N
    s_d = host(s).astype(np.float64)
    _, s_ref = _check_lite(host(losses), float(host(alpha)[0]), W, S_full, xm, 4, 128, False, s_d)
    assert np.all(np.abs(s_d - s_ref) <= 1e-5 * s_ref)
    rows = np.unique(np.linspace(0, ls.m - 1, 32).astype(int))
    clip = awq.awq_clip(W[rows], S_full, s_d, 4, 128)
    ci = host(cidx).astype(np.int64)[rows]
    chosen = np.take_along_axis(clip.errors, ci[:, :, None], axis=2)[:, :, 0]
    assert np.all(chosen <= clip.errors.min(axis=2) + 1e-4 * np.abs(clip.errors).max(axis=2))
    Ws = oracle.f32(W[rows] * s_d)
    amax = np.stack([np.abs(Ws[:, g0:g0 + 128]).max(axis=1) for g0 in range(0, n, 128)], axis=1)
    c_ref, s_ref2, z_ref = awq.quantize_groups(
        Ws, 4, 128, ranges=oracle.f32(amax * oracle.f32(awq.CLIP_RATIOS[ci])))
    assert np.array_equal(host(codes).astype(np.int64)[rows], c_ref)
    assert np.array_equal(host(scales).astype(np.float64)[rows], s_ref2)


def test_awq_layer_through_the_packed_product():
    """The AWQ-quantized layer runs on the packed format and the product as they
    are: codes of W diag(s) in groups of consecutive columns (gptq_pack, no
    permutation), activations X diag(1/s) (formed here on the host and rounded
    to bf16, as the previous operator would hand them over), and
    gptq_dequant_gemm gives X W_eff^T, W_eff = dequant(codes) diag(1/s) the
    oracle's effective weights, within the bf16 roundings of X/s and of the
    weights (2^-8 of each term, twice) and the fp32 sums."""
    q = need_gpu()
    rng = np.random.default_rng(21)
    m, n, tokens, bits, G = 256, 512, 2048, 4, 128
    W = synth.round_to_bf16((rng.standard_normal((m, n)) * 0.02).astype(np.float32)).astype(np.float64)
    X = rng.standard_normal((tokens, n))
    X[:, rng.choice(n, 5, replace=False)] *= 30.0
    X = synth.round_to_bf16(X.astype(np.float32)).astype(np.float64)
    say("awq layer product", m, n, tokens)
    r = _run(q, W, X, bits, G)
    codes = dev(r["codes"].astype(np.uint8), torch.uint8)
    packed = torch.empty((m, n * bits // 32), dtype=torch.int32, device="cuda")
    q.gptq_pack(codes, bits, packed)
    Xs = synth.round_to_bf16((X / r["s"]).astype(np.float32)).astype(np.float64)
    Y = torch.empty((64, m), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(q.gptq_dequant_gemm_workspace_size(64, m, n, False), 1), dtype=torch.uint8,
                     device="cuda")
    q.gptq_dequant_gemm(dev(Xs[:64].astype(np.float32), torch.bfloat16), packed, bits, G,
                        dev(r["scales"].astype(np.float32), torch.float32),
                        dev(r["zeros"].astype(np.float32), torch.float32), Y, ws=ws)
    torch.cuda.synchronize()
    W_eff = awq.dequant_groups(r["codes"], r["scales"], r["zeros"], G) / r["s"]
    Y_ref = X[:64] @ W_eff.T
    Wq = awq.dequant_groups(r["codes"], r["scales"], r["zeros"], G)
    bound = (2 * 2.0 ** -8 + 8 * np.sqrt(n) * EPS32) * (np.abs(Xs[:64]) @ np.abs(Wq).T) + 1e-6
    diff = np.abs(host(Y).astype(np.float64) - Y_ref)
    print(f"  max |Y - X W_eff^T| / bound {float((diff / bound).max()):.3f}", flush=True)
    assert np.all(diff <= bound)
