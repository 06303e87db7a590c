"""GPU parity: rtn_minmax and gptq_pack against the oracle, bit for bit."""
import numpy as np
import pytest

import oracle
from oracle.quantizer import f32
import synth

from gpu_util import dev, host, need_gpu, say, storage_dtype, torch

pytestmark = pytest.mark.gpu

RTN_CASES = [
    # m, n, G, bits, dtype, sym
    (64, 256, 128, 4, "bf16", False),
    (33, 1000, 64, 3, "f32", False),
    (17, 72, 8, 2, "bf16", False),
    (5, 300, 32, 8, "f32", False),
    (16, 4096, 128, 4, "bf16", False),
    (9, 130, -1, 4, "bf16", False),      # one group per row (workgroup path)
    (7, 200, 200, 3, "f32", False),      # group size off the wave path
    (11, 256, 128, 4, "bf16", True),
    (13, 96, 32, 3, "f32", True),
    (3, 1024, 512, 4, "bf16", False),
]


@pytest.mark.parametrize("m,n,G,bits,dt,sym", RTN_CASES)
def test_rtn_bit_exact(m, n, G, bits, dt, sym):
    q = need_gpu()
    rng = np.random.default_rng(m * 1000 + n)
    W = rng.standard_normal((m, n)) * 0.02
    W[:, :3] *= 20  # a few large values per row
    W = f32(W)
    if m > 2:
        W[1, :] = 0.0  # all-zero row: degenerate groups
    if dt == "bf16":
        W = synth.round_to_bf16(W.astype(np.float32)).astype(np.float64)
    codes_o, scales_o, zeros_o = oracle.rtn_minmax(W, bits, G, sym)
    Wd = dev(W.astype(np.float32), storage_dtype(dt))
    ng = scales_o.shape[1]
    codes = torch.empty((m, n), dtype=torch.uint8, device="cuda")
    scales = torch.empty((m, ng), dtype=torch.float32, device="cuda")
    zeros = torch.empty((m, ng), dtype=torch.float32, device="cuda")
    say("rtn", m, n, G, bits, dt, sym)
    q.rtn_minmax(Wd, bits, G, codes, scales, zeros, sym=sym)
    torch.cuda.synchronize()
    assert np.array_equal(host(codes).astype(np.int64), codes_o.astype(np.int64))
    assert np.array_equal(host(scales).astype(np.float64), scales_o)
    assert np.array_equal(host(zeros).astype(np.float64), zeros_o)


def test_rtn_strided_input():
    q = need_gpu()
    rng = np.random.default_rng(5)
    big = f32(rng.standard_normal((24, 320)) * 0.02)
    W = big[:, :256]
    codes_o, scales_o, zeros_o = oracle.rtn_minmax(W, 4, 64)
    Wd = dev(big.astype(np.float32), torch.float32)[:, :256]
    assert Wd.stride(0) == 320
    codes = torch.empty((24, 256), dtype=torch.uint8, device="cuda")
    scales = torch.empty((24, 4), dtype=torch.float32, device="cuda")
    zeros = torch.empty((24, 4), dtype=torch.float32, device="cuda")
    say("rtn strided")
    q.rtn_minmax(Wd, 4, 64, codes, scales, zeros)
    torch.cuda.synchronize()
    assert np.array_equal(host(codes), codes_o.astype(np.uint8))
    assert np.array_equal(host(scales).astype(np.float64), scales_o)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n", [1, 7, 33, 100, 4096])
def test_pack_bit_exact(bits, n):
    q = need_gpu()
    m = 6
    rng = np.random.default_rng(bits * 7919 + n)
    codes = rng.integers(0, 2 ** bits, (m, n)).astype(np.uint8)
    ref = oracle.pack_ref(codes, bits)
    nw = ref.shape[1]
    packed = torch.full((m, nw), -1, dtype=torch.int32, device="cuda")
    say("pack", bits, n)
    q.gptq_pack(dev(codes, torch.uint8), bits, packed)
    torch.cuda.synchronize()
    got = host(packed).view(np.uint32)
    assert np.array_equal(got, ref)
    assert np.array_equal(oracle.unpack_ref(got, n, bits), codes.astype(np.int64))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n", [1, 31, 100, 4096])
def test_pack_ordered_bit_exact(bits, n):
    """gptq_pack_ordered: row r's stream holds codes[r, perm[0]], codes[r, perm[1]], ...
    in the gptq_pack layout, bit for bit against the oracle's packing of the
    permuted codes."""
    q = need_gpu()
    m = 5
    rng = np.random.default_rng(bits * 31 + n)
    codes = rng.integers(0, 2 ** bits, (m, n)).astype(np.uint8)
    perm = rng.permutation(n).astype(np.int32)
    ref = oracle.pack_ref(codes[:, perm], bits)
    packed = torch.full((m, ref.shape[1]), -1, dtype=torch.int32, device="cuda")
    say("pack ordered", bits, n)
    q.gptq_pack_ordered(dev(codes, torch.uint8), bits, dev(perm, torch.int32), packed)
    torch.cuda.synchronize()
    assert np.array_equal(host(packed).view(np.uint32), ref)


def test_rtn_subnormal_groups_and_exact_half_steps():
    """Groups whose scale is subnormal (1 / scale overflows to inf in fp32) and
    groups whose values sit exactly on half steps of the grid (rounding ties):
    the codes still equal the oracle's rint(w / scale) decisions bit for bit."""
    q = need_gpu()
    rng = np.random.default_rng(11)
    m, n, G = 8, 256, 64
    W = f32(rng.standard_normal((m, n)) * 0.02)
    W[0, :] = f32(rng.standard_normal(n) * 1e-41)      # subnormal range: scale ~1e-43
    W[1, :64] = f32(rng.standard_normal(64) * 1e-44)   # a few subnormal steps only
    steps = np.arange(64) % 15 + 0.5                   # k + 1/2 on a unit grid
    W[2, 64:128] = steps
    W[2, 64] = 0.0
    W[2, 65] = 15.0                                    # range [0, 15]: scale 1, zero 0
    W[3, :64] = -steps * 0.25                          # scale 0.25, values on half steps
    W[3, 0] = -3.75
    W = W.astype(np.float32).astype(np.float64)
    for bits in (4, 3):
        codes_o, scales_o, zeros_o = oracle.rtn_minmax(W, bits, G)
        codes = torch.empty((m, n), dtype=torch.uint8, device="cuda")
        scales = torch.empty((m, n // G), dtype=torch.float32, device="cuda")
        zeros = torch.empty((m, n // G), dtype=torch.float32, device="cuda")
        say("rtn subnormal / half steps", bits)
        q.rtn_minmax(dev(W.astype(np.float32), torch.float32), bits, G, codes, scales, zeros)
        torch.cuda.synchronize()
        assert np.array_equal(host(scales).astype(np.float64), scales_o)
        assert np.array_equal(host(zeros).astype(np.float64), zeros_o)
        assert np.array_equal(host(codes).astype(np.int64), codes_o.astype(np.int64))
