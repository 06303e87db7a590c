"""GPU parity: gptq_hessian_accumulate and gptq_prepare against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from oracle.quantizer import f32

from gpu_util import dev, host, need_gpu, say, torch

pytestmark = pytest.mark.gpu

HESS_CASES = [
    # n, tokens, chunk, dtype
    (200, 300, 300, "bf16"),      # ragged tiles, one split
    (384, 8192, 2048, "bf16"),    # 3x3 tiles -> split over tokens (partials + reduce)
    (256, 1024, 1024, "f32"),     # fp32 activations (SIMT path)
    (130, 77, 77, "f32"),
    (1024, 4096, 2048, "bf16"),
    (1280, 8192, 2048, "bf16"),   # 5x5 tiles (row-major tile order), some tiles in half-length splits
    (2048, 16384, 2048, "bf16"),  # 8x8 tiles (super-tile order), some tiles in half-length splits
    (8192, 4096, 2048, "bf16"),   # 32x32 tiles: the region order in a split plan
]


def _x(n, tokens, chunk, dt, seed=0):
    wl = synth.custom_workload("hx", 8, n, tokens, chunk, x_dtype=dt, outlier_frac=0.02,
                               outlier_mult=30.0, workload_id=200 + seed)
    return synth.x_all(wl, "x")


@pytest.mark.parametrize("n,tokens,chunk,dt", HESS_CASES)
def test_hessian_lower_triangle(n, tokens, chunk, dt):
    q = need_gpu()
    X = _x(n, tokens, chunk, dt)
    S_ref = oracle.hessian_S([X])
    A_ref = oracle.hessian_S([np.abs(X)])  # sum |x_i x_j|, for the rounding bound
    S_l = torch.zeros((n, n), dtype=torch.float32, device="cuda")
    S_l += torch.triu(torch.full((n, n), 7.0, device="cuda"), 1)  # sentinel above the diagonal
    say("hessian", n, tokens, dt)
    q.gptq_hessian_accumulate(S_l, dev(X, torch.bfloat16 if dt == "bf16" else torch.float32))
    torch.cuda.synchronize()
    got = host(S_l).astype(np.float64)
    low = np.tril(np.ones((n, n), dtype=bool))
    # strict upper triangle untouched
    assert np.all(got[~low] == 7.0)
    err = np.abs(got - S_ref)[low]
    # fp32 accumulation (worst case): |err| <= (tokens + 8) * 2^-24 * sum_t |x_ti x_tj|
    bound = (tokens + 8) * 2.0 ** -24 * A_ref[low] + 1e-30
    assert np.all(err <= bound)
    assert err.max() <= 1e-5 * np.abs(S_ref).max()


def test_hessian_is_additive_over_calls():
    q = need_gpu()
    X = _x(256, 6144, 2048, "bf16", seed=3)
    Xd = dev(X, torch.bfloat16)
    S1 = torch.zeros((256, 256), dtype=torch.float32, device="cuda")
    S2 = torch.zeros((256, 256), dtype=torch.float32, device="cuda")
    say("hessian additive")
    q.gptq_hessian_accumulate(S1, Xd)
    for c in range(3):
        q.gptq_hessian_accumulate(S2, Xd[c * 2048:(c + 1) * 2048])
    torch.cuda.synchronize()
    S_ref = oracle.hessian_S([X])
    low = np.tril(np.ones((256, 256), dtype=bool))
    for S in (S1, S2):
        assert np.abs(host(S) - S_ref)[low].max() <= 1e-5 * np.abs(S_ref).max()


def test_hessian_long_token_axis_in_launches():
    """Many tiles (n = 16384: 2080 lower-triangle tiles) run unsplit, one
    launch per 65,536 tokens.  With 66,624 tokens (a second, short launch) S
    equals, bit for bit, two calls on tokens [0, 65536) and [65536, 66624), and
    sampled channel pairs agree with the fp64 sum within the fp32 accumulation
    bound."""
    q = need_gpu()
    n, tokens, split = 16384, 66624, 65536
    wl = synth.custom_workload("hlong", 8, n, tokens, 2082, outlier_frac=0.01,
                               outlier_mult=20.0, workload_id=230)
    X = synth.x_all(wl, "x")
    rng = np.random.default_rng(3)
    chans = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 62, replace=False)]))
    Xc = X[:, chans].astype(np.float64)
    S_ref = Xc.T @ Xc
    A_ref = np.abs(Xc).T @ np.abs(Xc)
    Xd = dev(X, torch.bfloat16)
    del X, Xc
    S1 = torch.zeros((n, n), dtype=torch.float32, device="cuda")
    S2 = torch.zeros((n, n), dtype=torch.float32, device="cuda")
    say("hessian long token axis", n, tokens)
    q.gptq_hessian_accumulate(S1, Xd)
    q.gptq_hessian_accumulate(S2, Xd[:split])
    q.gptq_hessian_accumulate(S2, Xd[split:])
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)
    got = host(S1)[np.ix_(chans, chans)].astype(np.float64)
    low = chans[:, None] >= chans[None, :]
    err = np.abs(got - S_ref)[low]
    bound = (tokens + 8) * 2.0 ** -24 * A_ref[low] + 1e-30
    assert np.all(err <= bound)


def test_hessian_deterministic():
    q = need_gpu()
    X = dev(_x(384, 8192, 2048, "bf16", seed=4), torch.bfloat16)
    outs = []
    say("hessian determinism")
    for _ in range(3):
        S = torch.zeros((384, 384), dtype=torch.float32, device="cuda")
        q.gptq_hessian_accumulate(S, X)
        outs.append(host(S))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


PREP_CASES = [
    # n, tokens, desc_act, perc_damp
    (256, 1024, False, 0.01),
    (200, 900, True, 0.01),      # ragged panels, desc_act
    (520, 4096, True, 0.01),     # several panels + ragged tail
    (64, 256, False, 0.1),
    (1, 10, False, 0.01),
    (130, 2048, False, 0.0),
    (4500, 9000, True, 0.01),    # trailing updates on the 128 x 128-tile product, ragged
    (8448, 9000, False, 0.01),   # the inverse's block-row products on it as well
    (16512, 4096, True, 0.01),   # inverse groups of 8 blocks, the last one ragged (1 block)
]


def _S_case(n, tokens, seed=0):
    X = _x(n, tokens, tokens, "bf16", seed=seed)
    return f32(oracle.hessian_S([X]))  # the fp32 S both sides start from


@pytest.mark.parametrize("n,tokens,desc,damp", PREP_CASES)
def test_prepare_matches_oracle(n, tokens, desc, damp):
    q = need_gpu()
    S = _S_case(n, tokens, seed=n)
    # perc_damp crosses the ABI as fp32: the oracle gets that same value
    P = oracle.prepare(S, float(np.float32(damp)), desc)
    Sd = dev(S.astype(np.float32), torch.float32)
    U = torch.empty((n, n), dtype=torch.float32, device="cuda")
    perm = torch.empty(n, dtype=torch.int32, device="cuda")
    dead = torch.empty(n, dtype=torch.uint8, device="cuda")
    lam = torch.empty(1, dtype=torch.float32, device="cuda")
    info = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    say("prepare", n, tokens, desc, damp)
    q.gptq_prepare(Sd, tokens, damp, desc, U, perm=perm, dead=dead, lambda_out=lam, info=info)
    torch.cuda.synchronize()
    assert int(host(info)[0]) == 0
    assert np.array_equal(host(perm), P.perm)
    assert np.array_equal(host(dead).astype(bool), P.dead)
    assert abs(float(host(lam)[0]) - P.lam) <= 2.0 ** -23 * abs(P.lam) + 1e-30
    Ug = host(U).astype(np.float64)
    assert np.all(np.tril(Ug, -1) == 0.0)
    # fp64 on both sides, rounded to fp32 on the device: within 2 ulp of fp32
    tol = 2.0 ** -22 * np.abs(P.U) + 1e-12 * np.abs(P.U).max()
    assert np.all(np.abs(Ug - P.U) <= tol)


def test_prepare_in_place_and_dead_columns():
    q = need_gpu()
    n = 192
    X = _x(n, 512, 512, "bf16", seed=11)
    X[:, [5, 77, 150]] = 0.0
    S = f32(oracle.hessian_S([X]))
    P = oracle.prepare(S, float(np.float32(0.01)), True)
    Sd = dev(S.astype(np.float32), torch.float32)
    perm = torch.empty(n, dtype=torch.int32, device="cuda")
    dead = torch.empty(n, dtype=torch.uint8, device="cuda")
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("prepare in place")
    q.gptq_prepare(Sd, 512, 0.01, True, Sd, perm=perm, dead=dead, info=info)  # U aliases S
    torch.cuda.synchronize()
    assert int(host(info)[0]) == 0
    assert np.flatnonzero(host(dead)).tolist() == [5, 77, 150]
    assert np.array_equal(host(perm), P.perm)
    Ug = host(Sd).astype(np.float64)
    assert np.all(np.abs(Ug - P.U) <= 2.0 ** -22 * np.abs(P.U) + 1e-12 * np.abs(P.U).max())


def test_prepare_reports_not_positive_definite():
    q = need_gpu()
    n = 96
    rng = np.random.default_rng(1)
    B = rng.standard_normal((n, n))
    S = f32(B + B.T)  # indefinite
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    U = torch.empty((n, n), dtype=torch.float32, device="cuda")
    say("prepare not-PD")
    q.gptq_prepare(dev(S.astype(np.float32), torch.float32), 10, 0.0, False, U, info=info)
    torch.cuda.synchronize()
    v = int(host(info)[0])
    assert 1 <= v <= n


@pytest.mark.parametrize("n,desc", [(64, False), (1280, True)])
def test_prepare_reports_non_finite(n, desc):
    """A NaN below the diagonal of S is reported (at n = 1280 with desc_act the
    permuted matrix is built through the symmetric copy and the row gather)."""
    q = need_gpu()
    S = _S_case(n, 256, seed=2)
    S[10, 3] = np.nan
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    U = torch.empty((n, n), dtype=torch.float32, device="cuda")
    say("prepare non-finite", n, desc)
    q.gptq_prepare(dev(S.astype(np.float32), torch.float32), 256, 0.01, desc, U, info=info)
    torch.cuda.synchronize()
    assert int(host(info)[0]) == -1


@pytest.mark.parametrize("n,desc", [(96, False), (1283, True)])
def test_prepare_reads_only_the_lower_triangle(n, desc):
    """NaN everywhere above S's diagonal changes nothing: info stays 0 and U is
    the oracle's (from the lower triangle alone).  n = 1283 with desc_act stages
    rows of the symmetric copy element by element (n not a multiple of 4)."""
    q = need_gpu()
    S = _S_case(n, 2048, seed=6)
    P = oracle.prepare(S, float(np.float32(0.01)), desc)
    S2 = S.astype(np.float32)
    S2[np.triu_indices(n, 1)] = np.nan
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    U = torch.empty((n, n), dtype=torch.float32, device="cuda")
    perm = torch.empty(n, dtype=torch.int32, device="cuda")
    say("prepare lower triangle only", n, desc)
    q.gptq_prepare(dev(S2, torch.float32), 2048, 0.01, desc, U, perm=perm, info=info)
    torch.cuda.synchronize()
    assert int(host(info)[0]) == 0
    assert np.array_equal(host(perm), P.perm)
    Ug = host(U).astype(np.float64)
    assert np.all(np.abs(Ug - P.U) <= 2.0 ** -22 * np.abs(P.U) + 1e-12 * np.abs(P.U).max())


def test_prepare_nan_on_diagonal_with_desc_act():
    """A NaN on S's diagonal with desc_act: info reports the non-finite input
    and the processing order is still a permutation (a NaN key orders as the
    smallest value, ties by index), so nothing downstream reads S or W through
    an unwritten perm slot."""
    q = need_gpu()
    n = 300
    S = _S_case(n, 512, seed=4)
    S[7, 7] = np.nan
    S[123, 123] = np.nan
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    U = torch.empty((n, n), dtype=torch.float32, device="cuda")
    perm = torch.full((n,), -5, dtype=torch.int32, device="cuda")
    say("prepare NaN diagonal desc_act", n)
    q.gptq_prepare(dev(S.astype(np.float32), torch.float32), 512, 0.01, True, U, perm=perm,
                   info=info)
    torch.cuda.synchronize()
    assert int(host(info)[0]) == -1
    p = host(perm).astype(np.int64)
    assert np.array_equal(np.sort(p), np.arange(n))
    d = np.diag(S).astype(np.float64)
    key = np.where(np.isnan(d), -np.inf, d)
    assert np.array_equal(p, np.argsort(-key, kind="stable"))
    assert p[-1] == 123 and p[-2] == 7  # the two NaN columns last, lower index first


def test_prepare_desc_act_order_with_exact_ties_over_several_chunks():
    """The order kernels sort chunks of 1024 columns and count by binary
    search in each: at n = 4500 (five chunks, the last ragged) with a diagonal
    of exactly tied values the device order equals the stable descending
    argsort bit for bit."""
    q = need_gpu()
    n = 4500
    rng = np.random.default_rng(9)
    dvals = rng.integers(1, 6, size=n).astype(np.float32)
    S = torch.from_numpy(np.diag(dvals)).cuda()
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    U = torch.empty((n, n), dtype=torch.float32, device="cuda")
    perm = torch.empty(n, dtype=torch.int32, device="cuda")
    say("prepare tied desc_act order", n)
    q.gptq_prepare(S, 1000, 0.01, True, U, perm=perm, info=info)
    torch.cuda.synchronize()
    assert int(host(info)[0]) == 0
    assert np.array_equal(host(perm).astype(np.int64), np.argsort(-dvals.astype(np.float64),
                                                                   kind="stable"))


def test_prepare_empty_calibration_is_refused():
    q = need_gpu()
    S = torch.zeros((8, 8), dtype=torch.float32, device="cuda")
    U = torch.empty((8, 8), dtype=torch.float32, device="cuda")
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(q.GPTQError) as ei:
        q.gptq_prepare(S, 0, 0.01, False, U, info=info)
    assert ei.value.status == 4


def test_prepare_from_concurrent_host_threads():
    """Two host threads run prepare on their own streams at once (the library's
    side streams are shared by the device): each U equals the one a single
    call gives, bit for bit (the factorization has a fixed order)."""
    import threading

    q = need_gpu()
    n, tokens = 640, 3000
    rng = np.random.default_rng(5)
    X = rng.standard_normal((tokens, n)).astype(np.float32)
    S = torch.zeros((n, n), dtype=torch.float32, device="cuda")
    q.gptq_hessian_accumulate(S, dev(X, torch.bfloat16))
    say("prepare concurrent", n)

    def run(stream, out):
        U = torch.empty((n, n), dtype=torch.float32, device="cuda")
        perm = torch.empty(n, dtype=torch.int32, device="cuda")
        info = torch.zeros(1, dtype=torch.int32, device="cuda")
        ws = torch.empty(q.gptq_prepare_workspace_size(n), dtype=torch.uint8, device="cuda")
        with torch.cuda.stream(stream):
            for _ in range(3):
                q.gptq_prepare(S, tokens, 0.01, True, U, perm=perm, info=info, ws=ws,
                               stream=stream)
        stream.synchronize()
        assert int(host(info)[0]) == 0
        out.append((host(U), host(perm)))

    ref = []
    run(torch.cuda.current_stream(), ref)
    outs = [[], []]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    threads = [threading.Thread(target=run, args=(streams[i], outs[i])) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    torch.cuda.synchronize()
    for o in outs:
        assert len(o) == 1
        assert np.array_equal(o[0][0], ref[0][0]) and np.array_equal(o[0][1], ref[0][1])
