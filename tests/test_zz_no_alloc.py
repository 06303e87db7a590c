"""GPU: gptq_quantize_layer_noalloc (the library's fixed per-GPU scratch, no
allocation) against gptq_quantize_layer (caller workspace), bit for bit, on two
calls in a row, the second with a smaller layer; and the refusal of a layer
whose workspace exceeds the scratch."""
import numpy as np
import pytest

import synth

from gpu_util import dev, host, need_gpu, say, torch

pytestmark = pytest.mark.gpu


def _prepared(q, wl):
    """U, perm and dead of the workload's layer from the device path itself."""
    ls = wl.layer()
    xs = wl.xs[ls.x]
    qs = wl.quant
    n = ls.n
    X = dev(synth.x_all(wl, ls.x), torch.bfloat16)
    S = torch.zeros((n, n), dtype=torch.float32, device="cuda")
    q.gptq_hessian_accumulate(S, X)
    U = torch.empty((n, n), dtype=torch.float32, device="cuda")
    perm = torch.empty(n, dtype=torch.int32, device="cuda")
    dead = torch.empty(n, dtype=torch.uint8, device="cuda")
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    q.gptq_prepare(S, xs.tokens, qs.perc_damp, qs.desc_act, U, perm=perm, dead=dead, info=info)
    torch.cuda.synchronize()
    assert int(host(info)[0]) == 0
    return U, perm, dead


def _outputs(q, m, n, G):
    ng = -(-n // G)
    return dict(codes=torch.full((m, n), 255, dtype=torch.uint8, device="cuda"),
                scales=torch.full((m, ng), -1.0, dtype=torch.float32, device="cuda"),
                zeros=torch.full((m, ng), -1.0, dtype=torch.float32, device="cuda"),
                g_idx=torch.full((n,), -1, dtype=torch.int32, device="cuda"),
                row_err=torch.full((m,), -1.0, dtype=torch.float32, device="cuda"),
                info=torch.full((1,), 7, dtype=torch.int32, device="cuda"))


def _compare(q, wl):
    ls = wl.layer()
    qs = wl.quant
    m, n = ls.m, ls.n
    U, perm, dead = _prepared(q, wl)
    W = dev(synth.weight(wl, ls.name), torch.bfloat16)
    cfg = q.make_config(qs.bits, qs.group_size, qs.block_size, qs.perc_damp, qs.desc_act)
    ref = _outputs(q, m, n, qs.group_size)
    q.gptq_quantize_layer(W, U, cfg, ref["codes"], ref["scales"], ref["zeros"], perm=perm,
                          dead=dead, g_idx=ref["g_idx"], row_err=ref["row_err"], info=ref["info"])
    out = _outputs(q, m, n, qs.group_size)
    say("no-alloc quantize", m, n, qs.group_size, qs.desc_act)
    q.gptq_quantize_layer_noalloc(W, U, cfg, out["codes"], out["scales"], out["zeros"], perm=perm,
                                  dead=dead, g_idx=out["g_idx"], row_err=out["row_err"],
                                  info=out["info"])
    torch.cuda.synchronize()
    for k in ref:
        a, b = host(ref[k]), host(out[k])
        assert np.array_equal(a, b), k
    assert int(host(out["info"])[0]) == 0
    assert host(out["codes"]).max() < 2 ** qs.bits


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    q = need_gpu()
    big = synth.custom_workload("noalloc_big", 1024, 2048, 4096, 2048, x_dist="laplace",
                                outlier_frac=0.0, bits=4, group_size=64, desc_act=True,
                                workload_id=601)
    small = synth.custom_workload("noalloc_small", 300, 640, 2048, 1024, x_dist="normal",
                                  outlier_frac=0.01, outlier_mult=20.0, bits=3, group_size=128,
                                  desc_act=False, workload_id=602)
    assert q.gptq_quantize_workspace_size(1024, 2048, q.make_config(4, 64, desc_act=True)) <= \
        q.GPTQ_NOALLOC_SCRATCH_BYTES
    _compare(q, big)
    _compare(q, small)


def test_noalloc_refuses_a_layer_beyond_its_scratch():
    q = need_gpu()
    m = n = 4096
    cfg = q.make_config(4, 128)
    W = torch.zeros((m, n), dtype=torch.bfloat16, device="cuda")
    U = torch.zeros((n, n), dtype=torch.float32, device="cuda")
    o = _outputs(q, m, n, 128)
    with pytest.raises(q.GPTQError) as ei:
        q.gptq_quantize_layer_noalloc(W, U, cfg, o["codes"], o["scales"], o["zeros"])
    assert ei.value.status == q.GPTQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert np.all(host(o["codes"]) == 255)  # nothing was enqueued
