"""GPU parity of the shared-row entry point (svd_select_and_verify_rows): row
pools with index tables, for the standard and the greedy rule.  Identity
indices must reproduce the dense entry points bit for bit (the statistics of a
pool row are computed by the same reduction); shared rows are checked against
the oracle on the gathered dense rows; indices outside a pool invalidate
exactly the prefixes that read them."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import check_ranges, host, require_gpu, say
from parity_harness import compare

pytestmark = pytest.mark.gpu


def _rows_call(svd, d, rule, temp, seed, row_base=0):
    out = svd.select_and_verify_rows(d["p_pool"], d["p_index"], d["q_pool"], d["q_index"],
                                     d["drafts"], rule=rule, temp_p=temp, seed=seed,
                                     row_base=row_base, want_alpha=True, want_scores=True)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("rule", ["standard", "greedy"])
@pytest.mark.parametrize("V,dt", [(3000, "bf16"), (1001, "bf16"), (777, "f32")])
def test_identity_indices_equal_the_dense_entry_points(rule, V, dt):
    svd = require_gpu()
    cfg = W.Config(70, "custom", B=5, K=3, gamma=6, V=V, dtype=dt, sigma0=1.0, sigma_step=0.0,
                   temp=0.8, boost=6.0, boost_prob=1.0)
    d = W.generate(cfg, device="cuda", data_seed=V)
    B, K, G = cfg.B, cfg.K, cfg.gamma
    pooled = {"p_pool": d["p"].reshape(-1, V), "q_pool": d["q"].reshape(-1, V),
              "p_index": torch.arange(B * K * (G + 1), dtype=torch.int32,
                                      device="cuda").reshape(B, K, G + 1),
              "q_index": torch.arange(B * K * G, dtype=torch.int32, device="cuda").reshape(B, K, G),
              "drafts": d["drafts"]}
    a = _rows_call(svd, pooled, rule, 0.8, 7, row_base=3)
    if rule == "greedy":
        b = host(svd.greedy_select_and_verify(d["p"], d["drafts"], temp_p=0.8, seed=7, row_base=3,
                                              want_alpha=True, want_scores=True))
    else:
        b = host(svd.select_and_verify(d["p"], d["q"], d["drafts"], temp_p=0.8, seed=7,
                                       row_base=3, want_alpha=True, want_scores=True))
    for k in ("selected", "accept_len", "next_token", "alpha", "scores"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def _gathered(d):
    pp, pi = W.to_host(d["p_pool"]), W.to_host(d["p_index"])
    qp, qi = W.to_host(d["q_pool"]), W.to_host(d["q_index"])
    return (np.ascontiguousarray(pp[pi]), np.ascontiguousarray(qp[qi]), W.to_host(d["drafts"]))


@pytest.mark.parametrize("rule", ["standard", "greedy"])
@pytest.mark.parametrize("V,B,K,G", [(5000, 6, 8, 16), (8193, 3, 4, 5), (600, 8, 8, 9)])
def test_shared_rows_match_oracle(orc, rule, V, B, K, G):
    svd = require_gpu()
    cfg = W.get_config("shared_marginal")
    say("rows", rule, V, B, K, G)
    d = W.generate_pooled(cfg, device="cuda", B=B, V=V, K=K, gamma=G, data_seed=V + B)
    assert d["q_pool"].shape[0] == B * G and d["p_pool"].shape[0] < B * K * (G + 1)
    g = _rows_call(svd, d, rule, cfg.temp, 5)
    check_ranges(g, K, G, V)
    hp, hq, hd = _gathered(d)
    rep = compare(orc, hp, hq, hd, g, cfg.temp, cfg.temp, 5, greedy=rule == "greedy")
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]
    assert rep.invalid == 0


@pytest.mark.parametrize("rule", ["standard", "greedy"])
def test_full_size_shared_marginal_sampled(orc, rule):
    svd = require_gpu()
    cfg = W.get_config("shared_marginal")
    d = W.generate_pooled(cfg, device="cuda")
    g = _rows_call(svd, d, rule, cfg.temp, cfg.seed)
    check_ranges(g, cfg.K, cfg.gamma, cfg.V)
    idx = [0, 7, 15]
    sub = {k: (v[idx] if k in ("p_index", "q_index", "drafts") else v) for k, v in d.items()
           if k in ("p_pool", "q_pool", "p_index", "q_index", "drafts")}
    hp, hq, hd = _gathered(sub)
    rep = compare(orc, hp, hq, hd, g, cfg.temp, cfg.temp, cfg.seed, prefixes=idx,
                  greedy=rule == "greedy")
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]


def test_indices_outside_the_pools(orc):
    svd = require_gpu()
    cfg = W.get_config("shared_marginal")
    d = W.generate_pooled(cfg, device="cuda", B=8, V=2000, K=3, gamma=4, data_seed=12)
    NP, NQ = d["p_pool"].shape[0], d["q_pool"].shape[0]
    pi, qi = d["p_index"].clone(), d["q_index"].clone()
    pi[1, 2, 1] = NP          # a scored verifier row past the pool
    qi[3, 0, 2] = -1          # a negative drafter row
    pi[5, :, 4] = NP + 1000  # every bonus row of prefix 5 (gamma = 4)
    bad = dict(d, p_index=pi, q_index=qi)
    g = _rows_call(svd, bad, "standard", cfg.temp, 2)
    hp_pool, hq_pool = W.to_host(d["p_pool"]), W.to_host(d["q_pool"])
    r = orc.select_and_verify_rows(hp_pool, W.to_host(pi), hq_pool, W.to_host(qi),
                                   W.to_host(d["drafts"]), temp_p=cfg.temp, seed=2)
    for k in ("selected", "accept_len", "next_token"):
        assert np.array_equal(g[k], getattr(r, k)), (k, g[k], getattr(r, k))
    assert g["accept_len"][1] == -1 and g["accept_len"][3] == -1


def test_host_side_errors():
    svd = require_gpu()
    cfg = W.get_config("shared_marginal")
    d = W.generate_pooled(cfg, device="cuda", B=2, V=512, K=2, gamma=3, data_seed=1)
    B, K, G, V = 2, 2, 3, 512
    NP, NQ = d["p_pool"].shape[0], d["q_pool"].shape[0]
    n = svd.svd_rows_workspace_bytes(B, K, G, V, NP, NQ)
    assert n > 0 and svd.svd_rows_workspace_bytes(B, K, G, V, 0, NQ) == 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(3)]

    def call(rule=0, np_=NP, nq=NQ, qix=d["q_index"], pix=d["p_index"], nbytes=n):
        return svd.svd_select_and_verify_rows(rule, d["p_pool"], np_, pix, d["q_pool"], nq, qix,
                                              d["drafts"], svd.SVD_BF16, B, K, G, V, 1.0, 1.0, 0,
                                              0, o[0], o[1], o[2], None, None, ws, nbytes, None)
    assert call(rule=2) == svd.SVD_EINVAL
    assert call(np_=0) == svd.SVD_EINVAL
    assert call(nq=0) == svd.SVD_EINVAL
    assert call(qix=None) == svd.SVD_EINVAL
    assert call(pix=None) == svd.SVD_EINVAL
    assert call(nbytes=n - 256) == svd.SVD_EWORKSPACE
    assert call(rule=1, nq=0, qix=None) == svd.SVD_OK
    torch.cuda.synchronize()
