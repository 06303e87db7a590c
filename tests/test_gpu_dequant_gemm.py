"""GPU parity: the dequantized-weight product and packing in processing order.

gptq_dequant_gemm is compared with the oracle's fp64 product on the same
seeded inputs in two ways:
  - against the kernel's own precision model, built here from the oracle's
    unpacked codes: each weight formed in fp32 as fma(q, s, -(z s)) and rounded
    to bf16, products exact, sums in fp64.  What is left is the order of the
    fp32 sums, bounded per output by 8 sqrt(n) 2^-24 sum_c |X_c w_c|;
  - against the exact product of the dequantized weights (oracle.dequant_matmul),
    where the bf16 rounding of each weight adds at most 2^-8 |X_c w_c| per term
    (half a unit in the last of its 8 significant bits).
Sizes span several tiles with ragged token, row and column tails, every width
2..8, group sizes from 8 to a whole row, the column permutation of desc_act,
decode batches (split K) and bf16 output; the full-size cases use the weight
shapes of the Llama-7B attention and MLP and the 70B projections.
"""
import numpy as np
import pytest

import oracle
import synth

from gpu_util import dev, host, need_gpu, say, torch

pytestmark = pytest.mark.gpu

EPS32 = 2.0 ** -24


def _bf16_rne(a32: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _weights_model(codes_p, scales, zeros, G):
    """Kernel precision model of W_q in processing order: bf16(fma(q, s, -(z s)))."""
    m, n = codes_p.shape
    g = np.arange(n) // G if G > 0 else np.zeros(n, dtype=np.int64)
    s32 = scales.astype(np.float32)[:, g]
    nzs = -(zeros.astype(np.float32)[:, g] * s32)  # fp32 product, as on the device
    f = (codes_p.astype(np.float64) * s32.astype(np.float64) + nzs.astype(np.float64))
    return _bf16_rne(f.astype(np.float32)).astype(np.float64)


def _inputs(rng, tokens, m, n, bits, G, perm_on):
    ng = 1 if G <= 0 else -(-n // G)
    codes = rng.integers(0, 2 ** bits, (m, n))
    scales = (rng.uniform(0.5, 2.0, (m, ng)) * 0.02 / (2 ** bits)).astype(np.float32)
    zeros = rng.integers(0, 2 ** bits, (m, ng)).astype(np.float32)
    X = synth.round_to_bf16(rng.standard_normal((tokens, n)).astype(np.float32))
    X[:, :: max(1, n // 7)] *= 20.0  # a few outlier channels
    X = synth.round_to_bf16(X.astype(np.float32))
    perm = rng.permutation(n).astype(np.int64) if perm_on else np.arange(n)
    return codes, scales, zeros, X, perm


def _run(q, X, codes, scales, zeros, perm, bits, G, perm_on, ydt=torch.float32, ldx=None):
    """codes in ORIGINAL column order; packs in processing order on the device."""
    tokens, n = X.shape
    m = codes.shape[0]
    if ldx is not None and ldx != n:
        Xbig = np.zeros((tokens, ldx), dtype=np.float32)
        Xbig[:, :n] = X
        Xbig[:, n:] = np.nan  # columns past n must not be read into the sums
        Xd = dev(Xbig, torch.bfloat16)[:, :n]
    else:
        Xd = dev(X, torch.bfloat16)
    nw = -(-(n * bits) // 32)
    cd = dev(codes.astype(np.uint8), torch.uint8)
    pd = dev(perm.astype(np.int32), torch.int32) if perm_on else None
    packed = torch.empty((m, nw), dtype=torch.int32, device="cuda")
    q.gptq_pack_ordered(cd, bits, pd, packed)
    Y = torch.empty((tokens, m), dtype=ydt, device="cuda")
    q.gptq_dequant_gemm(Xd, packed, bits, G, dev(scales, torch.float32),
                        dev(zeros, torch.float32), Y, perm=pd)
    torch.cuda.synchronize()
    return host(Y.float()).astype(np.float64), host(packed).view(np.uint32)


def _check(Y, X, codes, scales, zeros, perm, bits, G, rows=None, ybf16=False):
    n = X.shape[1]
    rows = np.arange(codes.shape[0]) if rows is None else rows
    c_p = codes[rows][:, perm]
    Xp = X.astype(np.float64)[:, perm]
    Wm = _weights_model(c_p, scales[rows], zeros[rows], G)
    Ym = Xp @ Wm.T
    mag = np.abs(Xp) @ np.abs(Wm).T
    tight = 8.0 * np.sqrt(n) * EPS32 * mag + 1e-30
    if ybf16:  # the output's own rounding to bf16 adds half a unit in its last place
        tight = (1 + 2.0 ** -8) * tight + 2.0 ** -8 * np.abs(Ym)
    err = np.abs(Y[:, rows] - Ym)
    print(f"  max err / tight bound {float((err / tight).max()):.3f}, "
          f"max rel to sum|Xw| {float((err / np.maximum(mag, 1e-30)).max()):.2e}", flush=True)
    assert np.all(err <= tight)
    # the exact product of the dequantized weights (original order, g_idx)
    pos = np.empty(n, dtype=np.int64)
    pos[perm] = np.arange(n)
    g_idx = pos // G if G > 0 else np.zeros(n, dtype=np.int64)
    packed_orig = oracle.pack_ref(codes[rows], bits)
    Yo = oracle.dequant_matmul(X, packed_orig, n, bits, scales[rows].astype(np.float64),
                               zeros[rows].astype(np.float64), g_idx)
    Wo = oracle.dequant_weights(packed_orig, n, bits, scales[rows].astype(np.float64),
                                zeros[rows].astype(np.float64), g_idx)
    loose = 2.0 ** -8 * (np.abs(X) @ np.abs(Wo).T) + tight
    assert np.all(np.abs(Y[:, rows] - Yo) <= loose)


CASES = [
    # tokens, m, n, bits, G, perm, ldx
    (300, 200, 520, 4, 128, False, None),   # 2 token tiles (256), ragged rows and columns
    (77, 130, 1000, 3, 64, True, None),     # 128-token tiles, desc_act permutation
    (16, 96, 4096, 4, 128, False, None),    # decode batch: split K, partial sums
    (1, 300, 2048, 3, 128, True, None),     # one token
    (33, 64, 256, 2, 16, False, None),      # 2 groups per 32-code run
    (40, 70, 384, 5, 8, True, None),        # 5-bit codes straddle words
    (260, 128, 192, 6, 24, False, None),    # group size not a power of two
    (5, 50, 640, 7, 40, False, None),       # group boundaries inside a run
    (129, 33, 136, 8, -1, True, None),      # one group per row
    (64, 80, 203, 4, 8, False, 208),        # n not a multiple of 8; NaN past n
    (3, 17, 77, 3, 32, True, None),         # tiny, one partial chunk
    # 256-token tiles fed by LDS DMA (n % 8 == 0, G a multiple of 64 or a whole row)
    (257, 129, 4160, 3, 128, False, None),  # one row and one token past a tile
    (200, 64, 136, 2, -1, True, None),      # whole-row group, permuted, partial chunk
    (513, 300, 1000, 5, 64, True, None),    # 3 token tiles, 40-column last chunk
    (384, 256, 2048, 6, 128, False, None),  # K split across workgroups
    # up to 16 tokens over a K past 8192 (the wide-K decode kernel)
    (16, 200, 8448, 3, 64, False, None),    # 3-bit (8-byte code loads), ragged rows
    (5, 130, 9216, 5, 128, True, None),     # 5-bit, permuted, 5 tokens
    (16, 64, 8704, 2, -1, False, None),     # 2-bit, one group per row, many K splits
    (1, 96, 16384, 6, 192, False, None),    # 6-bit, group 192, one token
    # >= 1024 tokens over >= 256 output tiles: weights dequantized once, dense product
    (1100, 13100, 264, 3, 8, True, None),   # ragged tokens, rows and last chunk; permuted
]


@pytest.mark.parametrize("tokens,m,n,bits,G,perm_on,ldx", CASES)
def test_dequant_gemm_parity(tokens, m, n, bits, G, perm_on, ldx):
    q = need_gpu()
    rng = np.random.default_rng(tokens * 7919 + m * 31 + n + bits)
    codes, scales, zeros, X, perm = _inputs(rng, tokens, m, n, bits, G, perm_on)
    say("dequant_gemm", tokens, m, n, bits, G, perm_on, ldx)
    Y, packed = _run(q, X, codes, scales, zeros, perm, bits, G, perm_on, ldx=ldx)
    # the processing-order packing, bit for bit
    assert np.array_equal(packed, oracle.pack_ref(codes[:, perm], bits))
    _check(Y, X, codes, scales, zeros, perm, bits, G)


@pytest.mark.parametrize("tokens", [2, 200])
def test_dequant_gemm_bf16_output(tokens):
    q = need_gpu()
    rng = np.random.default_rng(11 + tokens)
    m, n, bits, G = 150, 768, 4, 128
    codes, scales, zeros, X, perm = _inputs(rng, tokens, m, n, bits, G, False)
    say("dequant_gemm bf16 out", tokens, m, n)
    Y, _ = _run(q, X, codes, scales, zeros, perm, bits, G, False, ydt=torch.bfloat16)
    _check(Y, X, codes, scales, zeros, perm, bits, G, ybf16=True)


def test_dequant_gemm_wide_k_unsplit_bf16():
    """16 tokens over a K past 8192 with 32768 weight rows: the wide-K decode
    kernel runs without a K split (256 row blocks fill the GPU) and rounds its
    sums to bf16 itself; checked on sampled rows, every token."""
    q = need_gpu()
    rng = np.random.default_rng(77)
    m, n, bits, G, tokens = 32768, 8448, 4, 64, 16
    ng = n // G
    codes = rng.integers(0, 2 ** bits, (m, n), dtype=np.uint8)
    scales = (rng.uniform(0.5, 2.0, (m, ng)) * 0.02 / (2 ** bits)).astype(np.float32)
    zeros = rng.integers(0, 2 ** bits, (m, ng)).astype(np.float32)
    X = synth.round_to_bf16(rng.standard_normal((tokens, n)).astype(np.float32))
    perm = np.arange(n)
    say("dequant_gemm wide K unsplit", tokens, m, n)
    Y, _ = _run(q, X, codes, scales, zeros, perm, bits, G, False, ydt=torch.bfloat16)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 30, replace=False)]))
    _check(Y, X, codes.astype(np.int64), scales, zeros, perm, bits, G, rows=rows, ybf16=True)


def test_dequant_gemm_deterministic():
    q = need_gpu()
    rng = np.random.default_rng(12)
    tokens, m, n, bits, G = 8, 512, 2048, 4, 128
    codes, scales, zeros, X, perm = _inputs(rng, tokens, m, n, bits, G, True)
    say("dequant_gemm determinism")
    Y1, _ = _run(q, X, codes, scales, zeros, perm, bits, G, True)
    Y2, _ = _run(q, X, codes, scales, zeros, perm, bits, G, True)
    assert np.array_equal(Y1, Y2)


def test_device_gptq_output_feeds_dequant_gemm():
    """A layer quantized on the device (desc_act) -> packed in processing order ->
    product, against the oracle's product of the device's codes, scales, zeros and
    g_idx in original column order."""
    q = need_gpu()
    from post_weight_quantization_22_amd import pipeline

    rng = np.random.default_rng(13)
    m, n, tokens_cal, bits, G = 96, 384, 1024, 4, 64
    W = synth.round_to_bf16((rng.standard_normal((m, n)) * 0.02).astype(np.float32))
    Xc = synth.round_to_bf16(rng.standard_normal((tokens_cal, n)).astype(np.float32))
    Xc[:, 5] *= 20.0
    Xc = synth.round_to_bf16(Xc.astype(np.float32))
    cfg = q.make_config(bits, G, 128, 0.01, True, False)
    buf = pipeline.allocate(m, n, cfg, tokens_cal)
    say("device gptq -> dequant_gemm", m, n)
    pipeline.run_layer(buf, dev(W, torch.bfloat16), [dev(Xc, torch.bfloat16)])
    torch.cuda.synchronize()
    pipeline.check_info(buf)
    codes = host(buf.codes).astype(np.int64)
    scales = host(buf.scales).astype(np.float64)
    zeros = host(buf.zeros).astype(np.float64)
    g_idx = host(buf.g_idx).astype(np.int64)
    perm = host(buf.perm).astype(np.int64)
    assert np.array_equal(g_idx[perm], np.arange(n) // G)
    nw = -(-(n * bits) // 32)
    packed = torch.empty((m, nw), dtype=torch.int32, device="cuda")
    q.gptq_pack_ordered(buf.codes, bits, buf.perm, packed)
    X = synth.round_to_bf16(rng.standard_normal((37, n)).astype(np.float32))
    Y = torch.empty((37, m), dtype=torch.float32, device="cuda")
    q.gptq_dequant_gemm(dev(X, torch.bfloat16), packed, bits, G, buf.scales, buf.zeros, Y,
                        perm=buf.perm)
    torch.cuda.synchronize()
    Yd = host(Y).astype(np.float64)
    Yo = oracle.dequant_matmul(X, oracle.pack_ref(codes, bits), n, bits, scales, zeros, g_idx)
    Wo = oracle.dequant_weights(oracle.pack_ref(codes, bits), n, bits, scales, zeros, g_idx)
    bound = (2.0 ** -8 + 8.0 * np.sqrt(n) * EPS32) * (np.abs(X) @ np.abs(Wo).T)
    assert np.all(np.abs(Yd - Yo) <= bound)
    # and the product approximates the unquantized layer's
    Yw = X.astype(np.float64) @ W.astype(np.float64).T
    rel = np.linalg.norm(Yd - Yw) / np.linalg.norm(Yw)
    print(f"  ||X W_q^T - X W^T|| / ||X W^T|| = {rel:.3e}", flush=True)
    assert rel < 0.2


def test_static_groups_feed_the_product_without_a_permutation():
    """With static groups and desc_act the groups are runs of original columns:
    the codes are packed in original order and the product needs no gather."""
    q = need_gpu()
    from post_weight_quantization_22_amd import pipeline

    rng = np.random.default_rng(14)
    m, n, tokens_cal, bits, G = 80, 512, 1024, 4, 64
    W = synth.round_to_bf16((rng.standard_normal((m, n)) * 0.02).astype(np.float32))
    Xc = synth.round_to_bf16(rng.standard_normal((tokens_cal, n)).astype(np.float32))
    cfg = q.make_config(bits, G, 128, 0.01, True, False, static_groups=True)
    buf = pipeline.allocate(m, n, cfg, tokens_cal)
    say("static groups -> dequant_gemm", m, n)
    pipeline.run_layer(buf, dev(W, torch.bfloat16), [dev(Xc, torch.bfloat16)])
    torch.cuda.synchronize()
    pipeline.check_info(buf)
    g_idx = host(buf.g_idx).astype(np.int64)
    assert np.array_equal(g_idx, np.arange(n) // G)
    X = synth.round_to_bf16(rng.standard_normal((300, n)).astype(np.float32))
    Y = torch.empty((300, m), dtype=torch.float32, device="cuda")
    q.gptq_dequant_gemm(dev(X, torch.bfloat16), buf.packed, bits, G, buf.scales, buf.zeros, Y)
    torch.cuda.synchronize()
    codes = host(buf.codes).astype(np.int64)
    scales = host(buf.scales).astype(np.float64)
    zeros = host(buf.zeros).astype(np.float64)
    Yo = oracle.dequant_matmul(X, oracle.pack_ref(codes, bits), n, bits, scales, zeros, g_idx)
    Wo = oracle.dequant_weights(oracle.pack_ref(codes, bits), n, bits, scales, zeros, g_idx)
    bound = (2.0 ** -8 + 8.0 * np.sqrt(n) * EPS32) * (np.abs(X) @ np.abs(Wo).T)
    assert np.all(np.abs(host(Y).astype(np.float64) - Yo) <= bound)


FULL = [
    # name, m, n, bits, G, perm
    ("llama7b_attn", 4096, 4096, 4, 128, False),
    ("llama7b_gate_up", 11008, 4096, 4, 128, True),
    ("llama7b_down", 4096, 11008, 4, 128, True),
    ("llama70b_square", 8192, 8192, 3, 128, False),
    ("llama70b_down", 8192, 28672, 4, 64, True),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,m,n,bits,G,perm_on", FULL)
@pytest.mark.parametrize("tokens", [16, 2048])
def test_dequant_gemm_full_size(name, m, n, bits, G, perm_on, tokens):
    """Weight shapes of the layer workloads, one 2048-token sequence (prefill) and
    a 16-token decode batch; checked on 24 sampled weight rows, every token."""
    q = need_gpu()
    rng = np.random.default_rng(m + n + tokens)
    ng = -(-n // G)
    codes = rng.integers(0, 2 ** bits, (m, n), dtype=np.uint8)
    scales = (rng.uniform(0.5, 2.0, (m, ng)) * 0.02 / (2 ** bits)).astype(np.float32)
    zeros = rng.integers(0, 2 ** bits, (m, ng)).astype(np.float32)
    X = synth.round_to_bf16(rng.standard_normal((tokens, n)).astype(np.float32))
    perm = rng.permutation(n).astype(np.int64) if perm_on else np.arange(n)
    say("dequant_gemm full size", name, tokens, m, n, bits, G, perm_on)
    Y, _ = _run(q, X, codes, scales, zeros, perm, bits, G, perm_on)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 22, replace=False)]))
    _check(Y, X, codes.astype(np.int64), scales, zeros, perm, bits, G, rows=rows)


@pytest.mark.parametrize("tokens,n,ldx,ldxp", [
    (67, 4096, 4096, 4096),      # rows staged in LDS (n <= 16384, >= 64 tokens)
    (64, 11008, 11016, 11008),   # row stride past n
    (70, 20000, 20000, 20008),   # the 32768-position LDS variant, zeroed tail of Xp
    (3, 77, 77, 80),             # n not a multiple of 8: the per-element gather
    (16, 28672, 28672, 28672),   # a decode batch: the per-element gather
    (1000, 256, 256, 256),       # many rows per workgroup
])
def test_gather_columns_exact(tokens, n, ldx, ldxp):
    """gptq_gather_columns: Xp[t, p] = X[t, perm[p]] bit for bit, zeros past n."""
    q = need_gpu()
    rng = np.random.default_rng(tokens * 7 + n)
    X = rng.standard_normal((tokens, ldx)).astype(np.float32)
    perm = rng.permutation(n).astype(np.int32)
    say("gather", tokens, n, ldx, ldxp)
    Xd = dev(X, torch.bfloat16)[:, :n]
    Xp = torch.full((tokens, ldxp), 7.0, dtype=torch.bfloat16, device="cuda")
    q.gptq_gather_columns(Xd, dev(perm, torch.int32), Xp[:, :n])
    torch.cuda.synchronize()
    Xb = host(Xd.view(torch.int16)).astype(np.int64)
    got = host(Xp.view(torch.int16)).astype(np.int64)
    assert np.array_equal(got[:, :n], Xb[:, perm])
    assert np.all(got[:, n:] == 0)


@pytest.mark.parametrize("m,n,bits,G", [(130, 512, 4, 128), (64, 392, 3, 8), (33, 2048, 2, -1),
                                        (7, 96, 8, 32), (256, 4096, 5, 64)])
def test_dequantize_matches_the_product_weights(m, n, bits, G):
    """gptq_dequantize writes bf16(fma(q, s, -(z s))) bit for bit (the weights
    every product kernel forms), from the oracle-packed codes."""
    q = need_gpu()
    rng = np.random.default_rng(m * 13 + n + bits)
    codes = rng.integers(0, 2 ** bits, size=(m, n)).astype(np.float64)
    ng = -(-n // G) if G > 0 else 1
    scales = rng.uniform(1e-3, 2e-2, size=(m, ng)).astype(np.float32)
    zeros = rng.integers(0, 2 ** bits, size=(m, ng)).astype(np.float32)
    packed = oracle.pack_ref(codes, bits).astype(np.uint32)
    say("dequantize", m, n, bits, G)
    W = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    q.gptq_dequantize(dev(packed.view(np.int32), torch.int32), bits, G, dev(scales, torch.float32),
                      dev(zeros, torch.float32), n, W)
    torch.cuda.synchronize()
    got = host(W.view(torch.int16)).astype(np.uint16)
    ref = _weights_model(codes, scales, zeros, G).astype(np.float32)
    ref_bits = (ref.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(got, ref_bits)


@pytest.mark.parametrize("tokens,m,n,ydt,pad", [(600, 300, 520, "f32", 0), (256, 128, 64, "f32", 0),
                                                (1000, 513, 4096, "bf16", 0),
                                                (17, 40, 136, "f32", 0), (300, 260, 264, "f32", 24)])
def test_gemm_bf16_against_fp64(tokens, m, n, ydt, pad):
    """gptq_gemm_bf16 against the fp64 product of the same bf16 operands, within
    the fp32 summation bound 8 sqrt(n) 2^-24 sum |x w| (plus half a bf16 unit
    of the result for bf16 output); ragged token, row and chunk tails."""
    q = need_gpu()
    rng = np.random.default_rng(tokens + m + n)
    X = synth.round_to_bf16(rng.standard_normal((tokens, n)).astype(np.float32)).astype(np.float64)
    W = synth.round_to_bf16((rng.standard_normal((m, n)) * 0.05).astype(np.float32)).astype(np.float64)
    say("gemm_bf16", tokens, m, n, ydt, pad)
    Y = torch.empty((tokens, m), dtype=torch.bfloat16 if ydt == "bf16" else torch.float32,
                    device="cuda")
    # pad > 0: operands as views into wider rows (row strides n + pad)
    Xw = np.zeros((tokens, n + pad), dtype=np.float32)
    Xw[:, :n] = X
    Ww = np.zeros((m, n + pad), dtype=np.float32)
    Ww[:, :n] = W
    q.gptq_gemm_bf16(dev(Xw, torch.bfloat16)[:, :n], dev(Ww, torch.bfloat16)[:, :n], Y)
    torch.cuda.synchronize()
    ref = X @ W.T
    bound = 8 * np.sqrt(n) * EPS32 * (np.abs(X) @ np.abs(W).T) + 1e-30
    if ydt == "bf16":
        bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)
    diff = np.abs(host(Y.float()).astype(np.float64) - ref)
    print(f"  max diff / bound {float((diff / bound).max()):.3f}", flush=True)
    assert np.all(diff <= bound)
