"""GPU parity of the greedy-acceptance entry points (alpha = p(x); a rejected
token is resampled from p with it zeroed) against the oracle's greedy mode,
on small and ragged shapes, at full workload sizes on sampled prefixes, and a
chi-square of the committed tokens at K = 4 (the rule keeps the verifier's law
under self-selection)."""
import numpy as np
import pytest
import torch
from scipy.special import softmax

import workloads as W
from gpu_util import check_ranges, gen, host, require_gpu, say
from parity_harness import compare
from stats_util import _chisq_p

pytestmark = pytest.mark.gpu

CASES = [
    # (B, K, gamma, V, dtype, temp)
    (1, 1, 4, 32, "f32", 1.0),
    (3, 1, 5, 1000, "bf16", 1.0),
    (3, 2, 3, 1001, "bf16", 0.7),        # odd V: element-wise path
    (2, 3, 7, 4099, "f32", 1.3),
    (5, 4, 6, 8192, "bf16", 0.7),
    (4, 3, 5, 8193, "bf16", 1.0),        # a rejected token in a second segment is possible
    (2, 8, 16, 20000, "bf16", 1.0),
    (3, 1, 70, 2048, "bf16", 1.0),
    (1, 64, 2, 512, "bf16", 2.0),
    (2, 2, 4096, 64, "f32", 1.0),        # gamma at its limit
    (800, 1, 2, 8193, "bf16", 1.0),      # drawn in segments of 8192
    (2, 1, 3, 70008, "bf16", 0.7),       # 69 segments of 1024
    (2, 1, 1, 1, "f32", 1.0),            # V = 1: p(x) = 1, always accepted
    (3, 2, 2, 2, "bf16", 1.0),
    (4, 2, 5, 9000, "bf16", 0.05),       # nearly one-hot rows: weights down to the exp's clamp
    (4, 2, 5, 9000, "bf16", 40.0),       # nearly uniform rows
]


def run_greedy(svd, d, temp, seed, row_base=0):
    out = svd.greedy_select_and_verify(d["p"], d["drafts"], temp_p=temp, seed=seed,
                                       row_base=row_base, want_alpha=True, want_scores=True)
    torch.cuda.synchronize()
    return host(out)


def host_pd(d, prefixes=None):
    if prefixes is None:
        return W.to_host(d["p"]), W.to_host(d["drafts"])
    idx = torch.as_tensor(list(prefixes), device=d["p"].device)
    return W.to_host(d["p"].index_select(0, idx)), W.to_host(d["drafts"].index_select(0, idx))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_K%d_G%d_V%d_%s" % c[:5])
@pytest.mark.parametrize("seed", [2, 20261203])
def test_small_shapes_match_oracle(orc, case, seed):
    svd = require_gpu()
    B, K, G, V, dt, T = case
    say("greedy case", case, "seed", seed)
    cfg = W.Config(96, "custom", B=B, K=K, gamma=G, V=V, dtype=dt, sigma0=1.0, sigma_step=0.02,
                   temp=T, boost=6.0, boost_prob=0.8)
    d = gen(cfg, data_seed=seed * 5 + V)
    g = run_greedy(svd, d, T, seed, row_base=seed % 3)
    check_ranges(g, K, G, V)
    hp, hd = host_pd(d)
    rep = compare(orc, hp, None, hd, g, T, T, seed, row_base=seed % 3, greedy=True)
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]
    assert rep.invalid == 0


def test_rejections_never_redraw_the_rejected_token(orc):
    svd = require_gpu()
    cfg = W.Config(95, "custom", B=300, K=2, gamma=4, V=64, dtype="bf16", sigma0=1.5,
                   sigma_step=0.0, temp=1.0, boost=3.0, boost_prob=1.0)
    d = gen(cfg, data_seed=3)
    g = run_greedy(svd, d, 1.0, 9)
    hd = W.to_host(d["drafts"])
    L, sel, tok = g["accept_len"], g["selected"], g["next_token"]
    rej = L < cfg.gamma
    assert rej.sum() > 100
    x = hd[np.arange(cfg.B), sel, np.minimum(L, cfg.gamma - 1)]
    assert np.all(tok[rej] != x[rej])
    rep = compare(orc, W.to_host(d["p"]), None, hd, g, 1.0, 1.0, 9, greedy=True)
    assert rep.ok(), rep.failures[:5]


def test_point_mass_rows(orc):
    # p one-hot at every drafted token: alpha = 1 and the whole window accepted
    svd = require_gpu()
    B, K, G, V = 6, 3, 4, 40
    rng = np.random.default_rng(4)
    drafts = rng.integers(0, V, (B, K, G)).astype(np.int32)
    zp = np.full((B, K, G + 1, V), -np.inf, np.float32)
    np.put_along_axis(zp[:, :, :G], drafts[..., None], 2.0, axis=-1)
    zp[:, :, G] = rng.standard_normal((B, K, V)).astype(np.float32)
    p = torch.from_numpy(zp).cuda()
    g = host(svd.greedy_select_and_verify(p, torch.from_numpy(drafts).cuda(), seed=5,
                                          want_alpha=True))
    assert np.all(g["alpha"] == 1.0) and np.all(g["accept_len"] == G)
    rep = compare(orc, zp, None, drafts, g, 1.0, 1.0, 5, greedy=True)
    assert rep.ok(), rep.failures


def test_verify_equals_select_with_one_draft():
    svd = require_gpu()
    cfg = W.Config(94, "custom", B=33, K=1, gamma=6, V=9000, dtype="bf16", sigma0=1.0,
                   sigma_step=0.0, temp=0.9, boost=6.0, boost_prob=1.0)
    d = gen(cfg, data_seed=8)
    a = host(svd.greedy_select_and_verify(d["p"], d["drafts"], temp_p=0.9, seed=4,
                                          want_alpha=True))
    b = host(svd.greedy_verify(d["p"][:, 0].contiguous(), d["drafts"][:, 0].contiguous(),
                               temp_p=0.9, seed=4, want_alpha=True))
    assert np.array_equal(a["accept_len"], b["accept_len"])
    assert np.array_equal(a["next_token"], b["next_token"])
    assert np.array_equal(a["alpha"][:, 0], b["alpha"])
    assert np.all(a["selected"] == 0)


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_full_size_workloads_sampled(orc, cid):
    svd = require_gpu()
    cfg = W.get_config(cid)
    say("greedy workload", cfg.name)
    d = gen(cfg)
    g = run_greedy(svd, d, cfg.temp, cfg.seed)
    check_ranges(g, cfg.K, cfg.gamma, cfg.V)
    rng = np.random.default_rng(cid)
    idx = sorted(rng.choice(cfg.B, size=min(cfg.B, 6), replace=False).tolist())
    hp, hd = host_pd(d, idx)
    # compare() reads the GPU outputs at each prefix's batch index
    rep = compare(orc, hp, None, hd, g, cfg.temp, cfg.temp, cfg.seed, prefixes=idx, greedy=True)
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]


def test_committed_tokens_follow_the_verifier_at_four_drafts():
    # 200k trials of a V = 32 window with K = 4 drafts from the drafter rows and
    # argmax self-selection: every committed position follows its verifier row
    svd = require_gpu()
    n, K, G, V = 200_000, 4, 4, 32
    rng = np.random.default_rng(5)
    zp = (rng.standard_normal((G + 1, V)) * 2.0).astype(np.float32)
    zq = (zp[:G] + rng.standard_normal((G, V))).astype(np.float32)
    drafts = np.empty((n, K, G), np.int32)
    for j in range(G):
        c = np.cumsum(softmax(zq[j].astype(np.float64)))
        drafts[:, :, j] = np.minimum(np.searchsorted(c / c[-1], rng.random((n, K)), side="right"),
                                     V - 1)
    p = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(zp, (n, K, G + 1, V)))).cuda()
    g = host(svd.greedy_select_and_verify(p, torch.from_numpy(drafts).cuda(), seed=11))
    L, sel, tok = g["accept_len"], g["selected"], g["next_token"]
    assert np.all(L >= 0) and len(np.unique(sel)) == K
    kept = drafts[np.arange(n), sel]
    pv = []
    for j in range(G + 1):
        m = L >= j
        y = np.where(L[m] == j, tok[m], kept[m, min(j, G - 1)])
        pv.append(_chisq_p(np.bincount(y, minlength=V), softmax(zp[j].astype(np.float64))))
    say("p-values", pv)
    assert min(pv) > 1e-3 / (G + 1), pv


@pytest.mark.parametrize("cid", [4, 3])
def test_full_size_greedy_with_accepted_runs(orc, cid):
    # V = 152064 with confident verifier rows: accepted runs, residual draws past
    # position 0 and bonus draws, on every prefix of the batch
    svd = require_gpu()
    cfg = W.get_config(cid)
    d = _confident(cfg, 77 + cid, mode_frac=0.85 if cfg.K == 1 else 0.95)
    g = run_greedy(svd, d, cfg.temp, cfg.seed)
    check_ranges(g, cfg.K, cfg.gamma, cfg.V)
    L = g["accept_len"]
    say("greedy confident", cfg.name, "mean L %.2f" % L.mean(), "bonus", int((L == cfg.gamma).sum()),
        "L histogram", np.bincount(L, minlength=cfg.gamma + 1).tolist())
    assert L.mean() > 1.0 and ((L > 0) & (L < cfg.gamma)).sum() > 0
    if cfg.K == 1:
        assert (L == cfg.gamma).sum() > 0  # bonus draws
    else:
        assert L.max() >= 5  # long accepted runs of the kept draft
    hp, hd = host_pd(d)
    rep = compare(orc, hp, None, hd, g, cfg.temp, cfg.temp, cfg.seed, greedy=True)
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]
    assert rep.excused_within(), rep.summary()


def _confident(cfg, seed, mode_frac):
    # the workload's rows with each verifier row's mode logit raised by a
    # further 2, 3, 4, 5 or 6 (so p(mode) spans about 0.2 to 0.99997 at T = 0.7),
    # and a fraction mode_frac of drafted tokens set to their row's mode
    d = gen(cfg)
    g = torch.Generator(device="cuda").manual_seed(seed)
    p = d["p"]
    mode = p.argmax(-1, keepdim=True)
    extra = torch.randint(2, 7, mode.shape, generator=g, device="cuda").float()
    p.scatter_(-1, mode, (p.gather(-1, mode).float() + extra).to(p.dtype))
    G = cfg.gamma
    take = torch.rand(d["drafts"].shape, generator=g, device="cuda") < mode_frac
    d["drafts"] = torch.where(take, mode[:, :, :G, 0].to(torch.int32), d["drafts"]).contiguous()
    return d
