"""GPU parity over seeded random shapes: 112 configurations drawn once from
three fixed generators (the third at full-size vocabularies, as are the last
sets of the windowed and shared-row cases), each run through the library and compared with the oracle on
every prefix (parity_harness rules: decisions exact unless flagged as a
near-tie, alpha, scores and beta within their tolerances).

The draws mix what the fixed cases take one at a time: prefix counts on both
sides of the split-row threshold (1024 scored positions) and of the small
draw segments (fewer than 768 pass workgroups of 8192 tokens), vocabularies
with and without 16-byte rows, fp32 and bf16 logits, distinct verifier and
drafter temperatures, both acceptance rules, and beta on some standard cases.
A second set takes the windowed entry point the same way: ragged windows, an
EOS token planted in the drafts, and early exit on one-draft cases.  A third
takes the shared-row entry point with random index tables into pools drawn
from the generated rows: shared rows, repeated rows and rows nobody reads.  The
last runs the causal-consistency path search (lattice, then a beam over it).
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import check_ranges, gen, host, host_inputs, require_gpu, say
from parity_harness import compare

pytestmark = pytest.mark.gpu

MAX_ELEMS = 3_000_000  # logits per case, so the oracle stays quick


def _cases(n=48, seed=2026, first=0, max_elems=MAX_ELEMS, large=False):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        V = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 5000)),
                            int(rng.integers(5000, 70000))]))
        if large:  # vocabularies at full size
            V = int(rng.integers(100000, 160001))
        if rng.random() < 0.4:
            V = max(8, V - V % 8)  # whole 16-byte rows (bf16)
        K = int(rng.choice([1, 1, 2, 3, 8]))
        G = int(rng.choice([1, 2, 4, 8, 16, 33]))
        B = int(rng.choice([1, 2, 5, 16, 48, 130]))
        while B > 1 and B * K * (G + 1) * V > max_elems:
            B //= 2
        if B * K * (G + 1) * V > max_elems:
            continue
        dt = "f32" if rng.random() < 0.3 else "bf16"
        tp = float(np.float32(rng.choice([0.4, 0.7, 1.0, 1.6])))
        tq = tp if rng.random() < 0.5 else float(np.float32(rng.choice([0.5, 0.9, 1.3])))
        rule = "greedy" if rng.random() < 0.3 else "standard"
        beta = rule == "standard" and tq == tp and rng.random() < 0.3
        out.append((first + len(out), B, K, G, V, dt, tp, tq, rule, beta))
    return out


CASES = (_cases() + _cases(48, seed=3037, first=48) +
         _cases(16, seed=6151, first=96, max_elems=30_000_000, large=True))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "c%d_B%d_K%d_G%d_V%d_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[8]))
def test_random_shapes_match_oracle(orc, case):
    svd = require_gpu()
    i, B, K, G, V, dt, tp, tq, rule, beta = case
    say("case", case)
    cfg = W.Config(120 + i, "custom", B=B, K=K, gamma=G, V=V, dtype=dt, sigma0=1.0,
                   sigma_step=0.03, temp=tp, boost=5.0, boost_prob=0.7)
    d = gen(cfg, data_seed=1000 + i)
    seed, row_base = 77 + i, 5 * i
    if rule == "greedy":
        out = svd.greedy_select_and_verify(d["p"], d["drafts"], temp_p=tp, seed=seed,
                                           row_base=row_base, want_alpha=True, want_scores=True)
    else:
        out = svd.select_and_verify(d["p"], d["q"], d["drafts"], temp_p=tp, temp_q=tq, seed=seed,
                                    row_base=row_base, want_alpha=True, want_beta=beta,
                                    want_scores=True)
    torch.cuda.synchronize()
    g = host(out)
    check_ranges(g, K, G, V)
    hp, hq, hd = host_inputs(d)
    rep = compare(orc, hp, hq, hd, g, tp, tq, seed, row_base=row_base, greedy=rule == "greedy")
    say(rep.summary())
    assert rep.prefixes == B
    assert rep.ok(), rep.failures[:5]
    assert rep.excused_within(), rep.summary()


def _window_cases(n=32, seed=4711, first=0, max_elems=MAX_ELEMS, large=False):
    # the windowed entry point: ragged windows, an EOS token planted in the
    # drafts, early exit (one draft per prefix) on half of the one-draft cases
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        V = int(rng.choice([int(rng.integers(2, 3000)), int(rng.integers(3000, 40000))]))
        if large:  # vocabularies at full size
            V = int(rng.integers(100000, 160001))
        if rng.random() < 0.5:
            V = max(8, V - V % 8)
        K = int(rng.choice([1, 1, 2, 4]))
        G = int(rng.choice([2, 5, 8, 12, 20]))
        B = int(rng.choice([1, 3, 20, 70, 300]))
        while B > 1 and B * K * (G + 1) * V > max_elems:
            B //= 2
        if B * K * (G + 1) * V > max_elems:
            continue
        dt = "f32" if rng.random() < 0.3 else "bf16"
        rule = "greedy" if rng.random() < 0.4 else "standard"
        ragged = rng.random() < 0.7
        use_eos = rng.random() < 0.6
        early = K == 1 and rng.random() < 0.5
        tq = 0.9 if rng.random() < 0.5 else 1.2
        out.append((first + len(out), B, K, G, V, dt, rule, ragged, use_eos, early, tq))
    return out


WINDOW_CASES = (_window_cases() + _window_cases(32, seed=5821, first=32) +
                _window_cases(12, seed=7607, first=64, max_elems=30_000_000, large=True))


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "w%d_B%d_K%d_G%d_V%d_%s_%s%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "_early" if c[9] else ""))
def test_random_windows_match_oracle(orc, case):
    svd = require_gpu()
    i, B, K, G, V, dt, rule, ragged, use_eos, early, tq = case
    say("window case", case)
    tp = 0.9
    cfg = W.Config(200 + i, "custom", B=B, K=K, gamma=G, V=V, dtype=dt, sigma0=0.8,
                   sigma_step=0.02, temp=tp, boost=5.0, boost_prob=0.8)
    d = gen(cfg, data_seed=3000 + i)
    rng = np.random.default_rng(i)
    gb = rng.integers(1, G + 1, B).astype(np.int32) if ragged else None
    hd = W.to_host(d["drafts"]).copy()
    eos = -1
    if use_eos:
        eos = int(np.bincount(hd.ravel(), minlength=V).argmax())
        hd[rng.random(hd.shape) < 0.1] = eos
        d["drafts"] = torch.from_numpy(hd).cuda()
    seed, row_base = 500 + i, 3 * i
    out = svd.verify_window(d["p"], d["q"], d["drafts"],
                            gamma_b=None if gb is None else torch.from_numpy(gb).cuda(), eos=eos,
                            rule=rule, early_exit=early, temp_p=tp, temp_q=tq, seed=seed,
                            row_base=row_base, want_alpha=True, want_scores=not early)
    torch.cuda.synchronize()
    g = host(out)
    ok = g["selected"] >= 0
    assert np.all((g["accept_len"][ok] >= 0) & (g["accept_len"][ok] <= G))
    assert np.all((g["next_token"][ok] >= -2) & (g["next_token"][ok] < V))
    if early:  # alpha is streamed only up to each prefix's first rejection: decisions only
        g = dict(g, alpha=None)
    win = dict(gamma_b=np.full(B, G, np.int32) if gb is None else gb, eos=eos)
    rep = compare(orc, W.to_host(d["p"]), W.to_host(d["q"]), hd, g, tp, tq, seed,
                  row_base=row_base, greedy=rule == "greedy", window=win)
    say(rep.summary())
    assert rep.prefixes == B
    assert rep.ok(), rep.failures[:5]
    assert rep.excused_within(), rep.summary()


def _pool_cases(n=24, seed=9090, first=0, max_elems=MAX_ELEMS, large=False):
    # the shared-row entry point: pools smaller or larger than the rows the
    # index tables read (shared rows, and rows nobody reads)
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        V = int(rng.choice([int(rng.integers(2, 3000)), int(rng.integers(3000, 60000))]))
        if large:  # vocabularies at full size
            V = int(rng.integers(100000, 160001))
        if rng.random() < 0.5:
            V = max(8, V - V % 8)
        K = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 3, 8, 16]))
        B = int(rng.choice([1, 4, 16, 60]))
        while B > 1 and B * K * (G + 1) * V > max_elems:
            B //= 2
        if B * K * (G + 1) * V > max_elems:
            continue
        share = float(rng.choice([0.3, 1.0, 1.5]))  # pool rows per indexed row
        dt = "f32" if rng.random() < 0.3 else "bf16"
        rule = "greedy" if rng.random() < 0.4 else "standard"
        tq = 0.8 if rng.random() < 0.5 else 1.1
        out.append((first + len(out), B, K, G, V, dt, rule, share, tq))
    return out


POOL_CASES = (_pool_cases() + _pool_cases(24, seed=9191, first=24) +
              _pool_cases(8, seed=9337, first=48, max_elems=30_000_000, large=True))


@pytest.mark.parametrize("case", POOL_CASES, ids=lambda c: "p%d_B%d_K%d_G%d_V%d_%s_%s" % c[:7])
def test_random_pools_match_oracle(orc, case):
    svd = require_gpu()
    i, B, K, G, V, dt, rule, share, tq = case
    say("pool case", case)
    tp = 0.8
    cfg = W.Config(300 + i, "custom", B=B, K=K, gamma=G, V=V, dtype=dt, sigma0=0.7,
                   sigma_step=0.0, temp=tp, boost=5.0, boost_prob=0.8)
    d = gen(cfg, data_seed=5000 + i)
    rng = np.random.default_rng(100 + i)
    prow, qrow = d["p"].reshape(-1, V), d["q"].reshape(-1, V)
    NP = max(1, int(prow.shape[0] * share))
    NQ = max(1, int(qrow.shape[0] * share))
    # pools drawn from the generated rows (repeats allowed), indices into them
    p_pool = prow[torch.from_numpy(rng.integers(0, prow.shape[0], NP)).cuda()].contiguous()
    q_pool = qrow[torch.from_numpy(rng.integers(0, qrow.shape[0], NQ)).cuda()].contiguous()
    pi = rng.integers(0, NP, (B, K, G + 1)).astype(np.int32)
    qi = rng.integers(0, NQ, (B, K, G)).astype(np.int32)
    seed, row_base = 900 + i, 11 * i
    out = svd.select_and_verify_rows(p_pool, torch.from_numpy(pi).cuda(), q_pool,
                                     torch.from_numpy(qi).cuda(), d["drafts"], rule=rule,
                                     temp_p=tp, temp_q=tq, seed=seed, row_base=row_base,
                                     want_alpha=True, want_scores=True)
    torch.cuda.synchronize()
    g = host(out)
    check_ranges(g, K, G, V)
    hpp, hqp = W.to_host(p_pool), W.to_host(q_pool)
    hp, hq = np.ascontiguousarray(hpp[pi]), np.ascontiguousarray(hqp[qi])
    rep = compare(orc, hp, hq, W.to_host(d["drafts"]), g, tp, tq, seed, row_base=row_base,
                  greedy=rule == "greedy")
    say(rep.summary())
    assert rep.prefixes == B
    assert rep.ok(), rep.failures[:5]
    assert rep.invalid == 0
    assert rep.excused_within(), rep.summary()


CUM_EPS = 1e-5   # a running sum this close to tau may cut either way
RANK_EPS = 1e-4  # expansions this close in score may rank either way


def _cps_cases(n=24, seed=31337, first=0, max_elems=MAX_ELEMS):
    # causal-consistency path search: the lattice (tau cut, M_max, EOS) and a
    # beam over it, on rows of the register, streamed and split forms
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        V = int(rng.choice([int(rng.integers(2, 2000)), int(rng.integers(2000, 160000))]))
        if rng.random() < 0.6:
            V = max(8, V - V % 8)
        G = int(rng.choice([1, 3, 8, 16, 20]))
        B = int(rng.choice([1, 2, 6, 16, 40]))
        while B > 1 and B * G * V > MAX_ELEMS:
            B //= 2
        if B * G * V > MAX_ELEMS:
            continue
        dt = "f32" if rng.random() < 0.3 else "bf16"
        tau = float(rng.choice([0.3, 0.6, 0.8, 0.95]))
        m_max = int(rng.choice([1, 3, 8, 15, 16]))
        beam = int(rng.choice([1, 2, 3, 8]))
        eos = int(rng.integers(0, V)) if rng.random() < 0.4 else -1
        tq = float(rng.choice([0.7, 1.0, 1.4]))
        out.append((first + len(out), B, G, V, dt, tau, m_max, beam, eos, tq))
    return out


CPS_CASES = _cps_cases() + _cps_cases(24, seed=27182, first=24)


@pytest.mark.parametrize("case", CPS_CASES, ids=lambda c: "s%d_B%d_G%d_V%d_%s_m%d_b%d" % (
    c[0], c[1], c[2], c[3], c[4], c[6], c[7]))
def test_random_path_searches_match_oracle(case):
    import oracle
    svd = require_gpu()
    i, B, G, V, dt, tau, m_max, beam, eos, tq = case
    say("cps case", case)
    rng = np.random.default_rng(7000 + i)
    z = (rng.standard_normal((B, G, V)) * 2.0).astype(np.float32)
    z[:, :, rng.integers(0, V, 3)] += 3.0
    if eos >= 0:  # EOS on top of a few rows
        for _ in range(max(1, B // 2)):
            b, j = int(rng.integers(0, B)), int(rng.integers(0, G))
            z[b, j, eos] = z[b, j].max() + 2.0
    t = torch.from_numpy(z)
    if dt == "bf16":
        t = t.to(torch.bfloat16)
        hz = t.view(torch.int16).numpy().view(np.uint16)
    else:
        hz = z
    gl = svd.cps_lattice(t.cuda(), temp_q=tq, tau=tau, m_max=m_max, eos=eos)
    g = host(gl)
    o = oracle.cps_lattice(hz, temp_q=tq, tau=tau, m_max=m_max, eos=eos)
    assert np.array_equal(g["len"], o["len"])
    for b in range(B):
        for j in range(G):
            n_g, n_o = int(g["n_cand"][b, j]), int(o["n_cand"][b, j])
            if n_g != n_o:
                assert o["cum_margin"][b, j] < CUM_EPS, (b, j, n_g, n_o)
            n = min(n_g, n_o)
            assert np.array_equal(g["cand"][b, j, :n], o["cand"][b, j, :n]), (b, j)
            lo = o["cand_logp"][b, j, :n]
            assert np.all(np.abs(g["cand_logp"][b, j, :n] - lo) <= 2e-6 * np.maximum(1, np.abs(lo)))
            assert np.all(g["cand"][b, j, n_g:] == -1)
    # the beam over each side's own lattice, compared where neither lattice nor
    # ranking sits within its tolerance of a tie
    f = (rng.standard_normal((B, G, m_max, m_max)) * 0.4).astype(np.float32)
    gb = host(svd.cps_beam(gl, torch.from_numpy(f).cuda(), lam=0.6, beam=beam))
    ob = oracle.cps_beam(o, f, lam=0.6, beam=beam)
    compared = 0
    for b in range(B):
        if np.min(o["cum_margin"][b]) < CUM_EPS or ob["rank_margin"][b] < RANK_EPS:
            continue
        compared += 1
        assert np.array_equal(gb["path_len"][b], ob["path_len"][b]), b
        assert np.array_equal(gb["paths"][b], ob["paths"][b]), b
        live = ob["path_len"][b] > 0
        assert np.allclose(gb["score"][b][live], ob["score"][b][live], atol=1e-3)
    assert compared >= B // 2
