"""GPU parity of the windowed entry point (svd_verify_window): ragged per-prefix
draft lengths, EOS-aware commits and early exit after the first rejection,
against the oracle's window mode."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import check_ranges, host, require_gpu, say
from parity_harness import compare

pytestmark = pytest.mark.gpu


def _inputs(B, K, G, V, dt, seed, temp=0.9, sigma=0.6):
    cfg = W.Config(60, "custom", B=B, K=K, gamma=G, V=V, dtype=dt, sigma0=sigma, sigma_step=0.0,
                   temp=temp, boost=6.0, boost_prob=1.0)
    return cfg, W.generate(cfg, device="cuda", data_seed=seed)


def _call(svd, d, rule, gamma_b, eos, early, temp, seed, row_base=0, scores=True):
    out = svd.verify_window(d["p"], d["q"], d["drafts"], gamma_b=gamma_b, eos=eos, rule=rule,
                            early_exit=early, temp_p=temp, seed=seed, row_base=row_base,
                            want_alpha=True, want_scores=scores)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("rule", ["standard", "greedy"])
def test_full_windows_equal_the_dense_entry_points(rule):
    svd = require_gpu()
    cfg, d = _inputs(6, 3, 7, 3000, "bf16", 4)
    a = _call(svd, d, rule, None, -1, False, cfg.temp, 5)
    if rule == "greedy":
        b = host(svd.greedy_select_and_verify(d["p"], d["drafts"], temp_p=cfg.temp, seed=5,
                                              want_alpha=True, want_scores=True))
    else:
        b = host(svd.select_and_verify(d["p"], d["q"], d["drafts"], temp_p=cfg.temp, seed=5,
                                       want_alpha=True, want_scores=True))
    for k in ("selected", "accept_len", "next_token", "alpha", "scores"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k


CASES = [
    # (B, K, gamma, V, dtype)
    (16, 1, 8, 2000, "bf16"),
    (12, 4, 6, 1001, "bf16"),   # element-wise path
    (9, 3, 10, 777, "f32"),
    (20, 2, 5, 8200, "bf16"),   # draws across two segments
]


@pytest.mark.parametrize("rule", ["standard", "greedy"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_K%d_G%d_V%d_%s" % c)
def test_ragged_eos_windows_match_oracle(orc, rule, case):
    svd = require_gpu()
    B, K, G, V, dt = case
    say("window", rule, case)
    cfg, d = _inputs(B, K, G, V, dt, seed=V + K)
    rng = np.random.default_rng(V)
    gb = rng.integers(1, G + 1, B).astype(np.int32)
    hd = W.to_host(d["drafts"]).copy()
    eos = int(np.bincount(hd.ravel(), minlength=V).argmax())  # a token drafted often
    hd[rng.random(hd.shape) < 0.15] = eos                     # and planted in places
    d["drafts"] = torch.from_numpy(hd).cuda()
    g = _call(svd, d, rule, torch.from_numpy(gb).cuda(), eos, False, cfg.temp, 3, row_base=7)
    ok = g["selected"] >= 0
    assert np.all((g["next_token"][ok] >= -2) & (g["next_token"][ok] < V))
    rep = compare(orc, W.to_host(d["p"]), W.to_host(d["q"]), hd, g, cfg.temp, cfg.temp, 3,
                  row_base=7, greedy=rule == "greedy", window=dict(gamma_b=gb, eos=eos))
    say(rep.summary(), "eos ends:", int(np.sum(g["next_token"] == -2)))
    assert rep.ok(), rep.failures[:5]
    assert rep.invalid == 0
    # alpha is NaN exactly past each draft's usable length
    for b in range(B):
        for k in range(K):
            hits = np.nonzero(hd[b, k, :gb[b]] == eos)[0]
            m = int(hits[0]) + 1 if len(hits) else int(gb[b])
            assert np.all(np.isnan(g["alpha"][b, k, m:])) and not np.any(np.isnan(g["alpha"][b, k, :m]))


def _chunk_ends(B, G, V, dt):
    """The early exit's chunks: J = ceil(512 / B) positions (at most G) for the
    first two, then twice the chunk before; when the chunks follow a live list
    (rows cut into at least two slices, fewer than 1024 row pairs per chunk of
    J), at most max(J, 1024 // B), so that a chunk of the whole batch fits the
    list's grid.  Returns J and the end of every chunk."""
    J = min(G, -(-512 // B))
    es = 2 if dt == "bf16" else 4
    unit = 16 // es if (V * es) % 16 == 0 else 1
    smax = max(1, (V // unit) // 512)
    cap = max(J, 1024 // B) if (B * J < 1024 and smax > 1) else G
    ends, j0, c = [], 0, 0
    while j0 < G:
        j0 += J if c < 2 else max(J, min(J << (c - 1), cap))
        ends.append(min(j0, G))
        c += 1
    return J, ends


@pytest.mark.parametrize("rule", ["standard", "greedy"])
@pytest.mark.parametrize("B,V,dt", [(300, 4096, "bf16"), (300, 20000, "bf16"), (300, 20000, "f32"),
                                    (300, 20001, "bf16"), (20, 20000, "bf16")])
def test_early_exit_equals_full_streaming(orc, rule, B, V, dt):
    # V = 4096 (bf16): a row is too short to cut, chunks stream whole rows, so
    # alpha is bitwise that of full streaming; V = 20000: chunks follow the
    # live list (whole rows for the first chunk, slices of the live rows
    # after it), alpha within the parity tolerance; V = 20001: the same on
    # the element-wise path; B = 20: one chunk of every position, in slices
    svd = require_gpu()
    G = 12
    say("early exit", rule, V, dt)
    cfg, d = _inputs(B, 1, G, V, dt, seed=9, sigma=1.2)
    gb = torch.from_numpy(np.random.default_rng(1).integers(4, G + 1, B).astype(np.int32)).cuda()
    a = _call(svd, d, rule, gb, 17, True, cfg.temp, 6, scores=False)
    b = _call(svd, d, rule, gb, 17, False, cfg.temp, 6, scores=False)
    for k in ("selected", "accept_len", "next_token"):
        assert np.array_equal(a[k], b[k]), k
    # every position up to the first rejection was streamed, with the same alpha,
    # and nothing past the chunk that holds it
    L = a["accept_len"]
    J, ends = _chunk_ends(B, G, V, dt)
    say("chunk ends", ends)
    hd = W.to_host(d["drafts"])
    for i in range(B):
        hits = np.nonzero(hd[i, 0, :int(gb[i])] == 17)[0]
        m = int(hits[0]) + 1 if len(hits) else int(gb[i])
        n = min(int(L[i]) + 1, m)
        if V == 4096:
            assert np.array_equal(a["alpha"][i, 0, :n], b["alpha"][i, 0, :n], equal_nan=True)
        else:
            assert np.all(np.abs(a["alpha"][i, 0, :n] - b["alpha"][i, 0, :n]) <= 1e-5)
        t = min(int(L[i]), m - 1)  # the position that ends the prefix's stream
        end = min(m, next(e for e in ends if e > t))
        assert not np.any(np.isnan(a["alpha"][i, 0, :end])), i
        assert np.all(np.isnan(a["alpha"][i, 0, end:])), i
    streamed = np.sum(~np.isnan(a["alpha"]))
    say("positions streamed with early exit: %d of %d" % (streamed, np.sum(~np.isnan(b["alpha"]))))
    if J < G:
        assert streamed < 0.8 * np.sum(~np.isnan(b["alpha"]))
    else:  # one chunk: every usable position is streamed
        assert streamed == np.sum(~np.isnan(b["alpha"]))
    # alpha past the chunk of the first rejection is not streamed (NaN): decisions only
    rep = compare(orc, W.to_host(d["p"]), W.to_host(d["q"]), W.to_host(d["drafts"]),
                  dict(a, alpha=None), cfg.temp, cfg.temp, 6, greedy=rule == "greedy",
                  window=dict(gamma_b=W.to_host(gb), eos=17))
    assert rep.ok(), rep.failures[:5]


def test_full_size_batched_serving_early_exit(orc):
    svd = require_gpu()
    cfg = W.get_config("batched_serving")
    d = W.generate(cfg, device="cuda")
    g = _call(svd, d, "standard", None, -1, True, cfg.temp, cfg.seed, scores=False)
    full = host(svd.select_and_verify(d["p"], d["q"], d["drafts"], temp_p=cfg.temp,
                                      seed=cfg.seed))
    for k in ("accept_len", "next_token"):
        assert np.array_equal(g[k], full[k]), k
    idx = list(range(256))
    hp, hq, hd = (W.to_host(d[k].index_select(0, torch.tensor(idx, device="cuda")))
                  for k in ("p", "q", "drafts"))
    rep = compare(orc, hp, hq, hd, dict(g, alpha=None), cfg.temp, cfg.temp, cfg.seed,
                  prefixes=idx, window=dict(gamma_b=None, eos=-1))
    assert rep.ok(), rep.failures


def test_windows_outside_their_range_and_argument_errors():
    svd = require_gpu()
    cfg, d = _inputs(5, 2, 4, 512, "bf16", seed=2)
    gb = torch.tensor([0, 1, 4, 5, -3], dtype=torch.int32, device="cuda")
    g = _call(svd, d, "standard", gb, -1, False, cfg.temp, 1)
    assert list(g["accept_len"][[0, 3, 4]]) == [-1, -1, -1] and np.all(g["accept_len"][[1, 2]] >= 0)
    B, K, G, V = 5, 2, 4, 512
    ws = svd.alloc_workspace(B, K, G, V, "cuda")
    o = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(3)]
    sc = torch.empty((B, K), dtype=torch.float32, device="cuda")

    def call(eos=-1, early=0, scores=None):
        return svd.svd_verify_window(0, d["p"], d["q"], d["drafts"], None, eos, early, svd.SVD_BF16,
                                     B, K, G, V, 1.0, 1.0, 0, 0, o[0], o[1], o[2], scores, None,
                                     ws, ws.numel(), None)
    assert call(eos=V) == svd.SVD_EINVAL
    assert call(early=1) == svd.SVD_EINVAL          # K = 2
    assert call(scores=sc) == svd.SVD_OK
    torch.cuda.synchronize()
