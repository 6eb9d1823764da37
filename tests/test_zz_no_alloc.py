"""svd_select_and_verify_noalloc through the C ABI: the same outputs as
svd_select_and_verify with a workspace of its own, bit for bit, on two calls in
a row (the second on a smaller input, so it runs on what the first left in the
shared scratch), then once more after a call of the workspace entry point; and
the oracle's parity rules on the smaller call."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import gen, host, host_inputs, require_gpu, say
from parity_harness import compare

pytestmark = pytest.mark.gpu

BIG = W.Config(97, "custom", B=96, K=2, gamma=6, V=60000, dtype="bf16", sigma0=1.0,
               sigma_step=0.0, temp=0.8, boost=8.0, boost_prob=1.0)
SMALL = W.Config(98, "custom", B=5, K=3, gamma=4, V=3001, dtype="f32", sigma0=1.0,
                 sigma_step=0.0, temp=1.0, boost=6.0, boost_prob=1.0)


def _outputs(cfg, dev):
    B, K, G = cfg.B, cfg.K, cfg.gamma
    return {"selected": torch.full((B,), 7, dtype=torch.int32, device=dev),
            "accept_len": torch.full((B,), 7, dtype=torch.int32, device=dev),
            "next_token": torch.full((B,), 7, dtype=torch.int32, device=dev),
            "scores": torch.full((B, K), 7.0, dtype=torch.float32, device=dev),
            "alpha": torch.full((B, K, G), 7.0, dtype=torch.float32, device=dev),
            "beta": torch.full((B, K, G), 7.0, dtype=torch.float32, device=dev)}


def _call(svd, cfg, d, seed, noalloc):
    dev = d["p"].device
    o = _outputs(cfg, dev)
    # shapes and element type checked on the host before any launch
    et = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    assert d["p"].dtype == et and d["q"].dtype == et and d["drafts"].dtype == torch.int32
    assert tuple(d["p"].shape) == (cfg.B, cfg.K, cfg.gamma + 1, cfg.V)
    assert tuple(d["q"].shape) == (cfg.B, cfg.K, cfg.gamma, cfg.V)
    assert tuple(d["drafts"].shape) == (cfg.B, cfg.K, cfg.gamma)
    code = svd.SVD_BF16 if et == torch.bfloat16 else svd.SVD_F32
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (d["p"], d["q"], d["drafts"], code, cfg.B, cfg.K, cfg.gamma, cfg.V, cfg.temp, cfg.temp,
            seed, 3, o["selected"], o["accept_len"], o["next_token"], o["scores"], o["alpha"],
            o["beta"])
    if noalloc:
        rc = svd.svd_select_and_verify_noalloc(*args, stream)
    else:
        ws = svd.alloc_workspace(cfg.B, cfg.K, cfg.gamma, cfg.V, dev)
        rc = svd.svd_select_and_verify(*args, ws, ws.numel(), stream)
    assert rc == svd.SVD_OK, svd.svd_strerror(rc)
    torch.cuda.synchronize()
    return host(o)


def _same(a, b, what):
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), (what, k)


def test_noalloc_equals_the_workspace_entry_point(orc):
    svd = require_gpu()
    big, small = gen(BIG, data_seed=11), gen(SMALL, data_seed=12)
    say("noalloc: first call B=%d K=%d gamma=%d V=%d bf16" % (BIG.B, BIG.K, BIG.gamma, BIG.V))
    n1 = _call(svd, BIG, big, 21, True)
    say("noalloc: second call, smaller, B=%d K=%d gamma=%d V=%d fp32"
        % (SMALL.B, SMALL.K, SMALL.gamma, SMALL.V))
    n2 = _call(svd, SMALL, small, 22, True)
    say("noalloc: reference calls with workspaces of their own")
    r1 = _call(svd, BIG, big, 21, False)
    r2 = _call(svd, SMALL, small, 22, False)
    _same(n1, r1, "first call")
    _same(n2, r2, "second call")
    say("noalloc: once more after the workspace calls")
    _same(_call(svd, BIG, big, 21, True), r1, "third call")
    # the smaller call also under the oracle's parity rules
    hp, hq, hd = host_inputs(small)
    rep = compare(orc, hp, hq, hd, n2, SMALL.temp, SMALL.temp, 22, row_base=3)
    say("noalloc parity:", rep.summary())
    assert rep.ok(), rep.failures


def test_noalloc_rejects_sizes_beyond_its_scratch():
    svd = require_gpu()
    # B = 2048 at gamma = 8, V = 152064 needs 32 MiB of workspace: refused on the
    # host, before any HIP call, with fake never-dereferenced addresses
    need = svd.svd_workspace_bytes(2048, 1, 8, 152064)
    assert need > svd.SVD_NOALLOC_SCRATCH_BYTES
    rc = svd.svd_select_and_verify_noalloc(4096, 8192, 12288, svd.SVD_BF16, 2048, 1, 8, 152064,
                                           1.0, 1.0, 0, 0, 16384, 20480, 24576, None, None, None,
                                           None)
    assert rc == svd.SVD_ESCRATCH


def test_noalloc_graph_replays():
    # a call captured in a HIP graph (through torch's graph API) after an eager
    # call on the device, replayed three times with eager calls of other sizes
    # and seeds in between (they leave their own contents in the shared
    # scratch): every replay gives the eager call's outputs bit for bit
    svd = require_gpu()
    cfg = W.Config(99, "custom", B=64, K=2, gamma=6, V=30000, dtype="bf16", sigma0=1.0,
                   sigma_step=0.0, temp=0.8, boost=8.0, boost_prob=1.0)
    d, other = gen(cfg, data_seed=31), gen(SMALL, data_seed=32)
    dev = d["p"].device
    o = _outputs(cfg, dev)
    code = svd.SVD_BF16

    def call():
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = svd.svd_select_and_verify_noalloc(
            d["p"], d["q"], d["drafts"], code, cfg.B, cfg.K, cfg.gamma, cfg.V, cfg.temp,
            cfg.temp, 41, 0, o["selected"], o["accept_len"], o["next_token"], o["scores"],
            o["alpha"], None, stream)
        assert rc == svd.SVD_OK
        return o

    torch.cuda.synchronize()
    ref = host(call())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        _call(svd, SMALL, other, 50 + r, True)  # eager, different sizes, same scratch
        g.replay()
        torch.cuda.synchronize()
        got = host(o)
        for k in ("selected", "accept_len", "next_token", "scores", "alpha"):
            assert np.array_equal(got[k], ref[k], equal_nan=True), (r, k)
        say("noalloc replay", r, "matches the eager call")
