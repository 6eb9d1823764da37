"""Behaviour of the C ABI on the GPU: equivalences, optional outputs, streams,
data errors and argument errors, all called through the ctypes binding."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import gen, host, host_inputs, require_gpu, say
from parity_harness import compare

pytestmark = pytest.mark.gpu

CFG = W.Config(96, "custom", B=6, K=1, gamma=6, V=5000, dtype="bf16", sigma0=1.0,
               sigma_step=0.0, temp=1.0, boost=6.0, boost_prob=1.0)


def test_verify_equals_select_with_one_draft():
    svd = require_gpu()
    d = gen(CFG, data_seed=3)
    a = svd.select_and_verify(d["p"], d["q"], d["drafts"], seed=5, want_alpha=True, want_beta=True)
    b = svd.verify(d["p"][:, 0].contiguous(), d["q"][:, 0].contiguous(),
                   d["drafts"][:, 0].contiguous(), seed=5, want_alpha=True, want_beta=True)
    torch.cuda.synchronize()
    assert torch.equal(a["accept_len"], b["accept_len"])
    assert torch.equal(a["next_token"], b["next_token"])
    assert torch.equal(a["alpha"][:, 0], b["alpha"])
    assert torch.equal(a["beta"][:, 0], b["beta"])
    assert torch.all(a["selected"] == 0)


def test_optional_outputs_do_not_change_results():
    svd = require_gpu()
    cfg = W.Config(95, "custom", B=5, K=4, gamma=5, V=3000, dtype="bf16", sigma0=1.5,
                   sigma_step=0.0, temp=1.0, boost=6.0, boost_prob=1.0)
    d = gen(cfg, data_seed=4)
    full = host(svd.select_and_verify(d["p"], d["q"], d["drafts"], seed=2, want_alpha=True,
                                      want_beta=True, want_scores=True))
    bare = host(svd.select_and_verify(d["p"], d["q"], d["drafts"], seed=2))
    for k in ("selected", "accept_len", "next_token"):
        assert np.array_equal(full[k], bare[k])


def test_non_default_stream_and_workspace_reuse():
    svd = require_gpu()
    d = gen(CFG, data_seed=6)
    ref = host(svd.select_and_verify(d["p"], d["q"], d["drafts"], seed=8))
    ws = svd.alloc_workspace(CFG.B, 1, CFG.gamma, CFG.V, d["p"].device)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(3):
            out = svd.select_and_verify(d["p"], d["q"], d["drafts"], seed=8, workspace=ws)
    s.synchronize()
    got = host(out)
    for k in ("selected", "accept_len", "next_token"):
        assert np.array_equal(ref[k], got[k])


def test_row_base_shifts_uniform_rows(orc):
    svd = require_gpu()
    d = gen(CFG, data_seed=7)
    g = host(svd.select_and_verify(d["p"], d["q"], d["drafts"], seed=1, row_base=12345,
                                   want_alpha=True))
    rep = compare(orc, *host_inputs(d), g, 1.0, 1.0, 1, row_base=12345)
    assert rep.ok(), rep.failures


@pytest.mark.parametrize("K,V,scores", [(2, 1000, True), (1, 20000, True), (1, 20000, False)])
def test_minus_inf_logits_and_data_errors(orc, K, V, scores):
    # (1, 20000): one draft per prefix, rows of three draw segments; without
    # scores the selection reads a single draft's alpha once
    svd = require_gpu()
    cfg = W.Config(94, "custom", B=8, K=K, gamma=4, V=V, dtype="f32", sigma0=1.0,
                   sigma_step=0.0, temp=1.0, boost=6.0, boost_prob=1.0)
    d = gen(cfg, data_seed=8)
    p, q, dr = d["p"], d["q"], d["drafts"]
    k = K - 1
    p[0, :, :, V // 2:] = -float("inf")       # legal: half the vocabulary has p = 0
    q[1, 0, 2, dr[1, 0, 2]] = -float("inf")   # q(x) = 0 -> alpha = 1
    p[2, k, 1, dr[2, k, 1]] = -float("inf")   # p(x) = 0 -> alpha = 0
    p[3, k, 2, 17] = float("nan")             # invalid
    q[4, 0, 0, 3] = float("inf")              # invalid
    dr[5, k, 3] = V                           # token out of range
    p[6, 0, 1, :] = -float("inf")             # all -inf row
    dr[7, 0, 0] = -5
    g = host(svd.select_and_verify(p, q, dr, seed=4, want_alpha=True, want_scores=scores))
    for b in (3, 4, 5, 6, 7):
        assert g["selected"][b] == -1 and g["accept_len"][b] == -1 and g["next_token"][b] == -1
    assert g["alpha"][1, 0, 2] == 1.0 and g["alpha"][2, k, 1] == 0.0
    rep = compare(orc, *host_inputs(d), g, 1.0, 1.0, 4)
    say(rep.summary())
    assert rep.ok(), rep.failures
    assert rep.invalid == 5


def test_invalid_bonus_row(orc):
    svd = require_gpu()
    cfg = W.Config(93, "custom", B=3, K=1, gamma=3, V=600, dtype="bf16", sigma0=1.0,
                   sigma_step=0.0, temp=1.0, boost=6.0, boost_prob=1.0)
    d = gen(cfg, data_seed=9)
    d["q"].copy_(d["p"][:, :, :3])            # alpha == 1: every prefix draws its bonus
    d["p"][1, 0, 3, 5] = float("nan")         # prefix 1's bonus row is invalid
    g = host(svd.select_and_verify(d["p"], d["q"], d["drafts"], seed=1))
    assert list(g["accept_len"]) == [3, -1, 3]
    assert g["next_token"][1] == -1 and g["selected"][1] == -1
    rep = compare(orc, *host_inputs(d), g, 1.0, 1.0, 1)
    assert rep.ok(), rep.failures


def test_identical_rows_accept_everything():
    svd = require_gpu()
    d = gen(CFG, data_seed=10)
    d["q"].copy_(d["p"][:, :, :CFG.gamma])
    g = host(svd.select_and_verify(d["p"], d["q"], d["drafts"], seed=3, want_alpha=True,
                                   want_beta=True, want_scores=True))
    assert np.all(g["alpha"] == 1.0)
    assert np.all(g["accept_len"] == CFG.gamma)
    assert np.allclose(g["beta"], 1.0, atol=1e-5)
    assert np.all(g["scores"] == CFG.gamma)


def test_argument_errors_through_the_abi():
    svd = require_gpu()
    d = gen(CFG, data_seed=11)
    B, G, V = CFG.B, CFG.gamma, CFG.V
    out = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(3)]
    ws = svd.alloc_workspace(B, 1, G, V, "cuda")
    n = ws.numel()
    st = torch.cuda.current_stream().cuda_stream
    args = dict(p=d["p"], q=d["q"], dr=d["drafts"])

    def call(**kw):
        a = dict(args, dtype=svd.SVD_BF16, B=B, K=1, G=G, V=V, tp=1.0, tq=1.0, ws=ws, n=n)
        a.update(kw)
        return svd.svd_select_and_verify(a["p"], a["q"], a["dr"], a["dtype"], a["B"], a["K"],
                                         a["G"], a["V"], a["tp"], a["tq"], 0, 0, out[0], out[1],
                                         out[2], None, None, None, a["ws"], a["n"], st)

    assert call() == svd.SVD_OK
    assert call(p=None) == svd.SVD_EINVAL
    assert call(dtype=7) == svd.SVD_EDTYPE
    assert call(B=0) == svd.SVD_EINVAL
    assert call(K=65) == svd.SVD_EINVAL
    assert call(tp=0.0) == svd.SVD_EINVAL
    assert call(tq=float("nan")) == svd.SVD_EINVAL
    assert call(tp=float("inf")) == svd.SVD_EINVAL
    assert call(n=n - 1) == svd.SVD_EWORKSPACE
    assert call(ws=ws.data_ptr() + 8) == svd.SVD_EINVAL
    torch.cuda.synchronize()
