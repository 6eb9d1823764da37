"""GPU parity of the causal-consistency path search (svd_cps_lattice,
svd_cps_beam) against the oracle: the candidate order is exact (it is the order
of the logits), the cut at tau is exact unless a running sum lies within
CUM_EPS of tau, log-probabilities agree to fp32 accuracy, and the beam paths
are exact unless two expansions' scores lie within RANK_EPS."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import host, require_gpu, say

pytestmark = pytest.mark.gpu

CUM_EPS = 1e-5
RANK_EPS = 1e-4


def _rows(seed, B, G, V, dt, scale=2.0, eos=-1, eos_at=()):
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((B, G, V)) * scale).astype(np.float32)
    z[:, :, rng.integers(0, V, 3)] += 3.0  # a few strong tokens
    for b, j in eos_at:
        z[b, j, eos] = z[b, j].max() + 2.0
    t = torch.from_numpy(z)
    if dt == "bf16":
        t = t.to(torch.bfloat16)
        host_z = t.view(torch.int16).numpy().view(np.uint16)
    else:
        host_z = z
    return t.cuda(), host_z


def _check_lattice(g, o, m_max):
    B, G = o["n_cand"].shape
    flagged = 0
    assert np.array_equal(g["len"], o["len"])
    for b in range(B):
        for j in range(G):
            n_g, n_o = int(g["n_cand"][b, j]), int(o["n_cand"][b, j])
            if n_g != n_o:
                assert o["cum_margin"][b, j] < CUM_EPS, (b, j, n_g, n_o, o["cum_margin"][b, j])
                flagged += 1
            n = min(n_g, n_o)
            assert np.array_equal(g["cand"][b, j, :n], o["cand"][b, j, :n])
            lo = o["cand_logp"][b, j, :n]
            assert np.all(np.abs(g["cand_logp"][b, j, :n] - lo) <= 2e-6 * np.maximum(1, np.abs(lo)))
            assert np.all(g["cand"][b, j, n_g:] == -1)
    return flagged


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("V,B,G,tau,m_max", [(1000, 4, 8, 0.8, 15), (1001, 3, 5, 0.5, 4),
                                             (37, 2, 6, 0.95, 16), (8, 2, 3, 0.99, 16),
                                             (20000, 2, 4, 0.8, 1)])
def test_lattice_matches_oracle(dt, V, B, G, tau, m_max):
    svd = require_gpu()
    say("lattice", dt, V, B, G, tau, m_max)
    q, hz = _rows(V + G, B, G, V, dt)
    g = host(svd.cps_lattice(q, temp_q=0.9, tau=tau, m_max=m_max))
    o = oracle.cps_lattice(hz, temp_q=0.9, tau=tau, m_max=m_max)
    assert _check_lattice(g, o, m_max) <= 1


def test_lattice_eos_and_invalid_rows():
    svd = require_gpu()
    q, hz = _rows(3, 4, 7, 500, "bf16", eos=11, eos_at=[(0, 2), (0, 5), (2, 6)])
    q[3, 1, 40] = float("nan")
    hz = hz.copy()
    hz[3, 1, 40] = 0x7FC0
    g = host(svd.cps_lattice(q, tau=0.8, m_max=15, eos=11))
    o = oracle.cps_lattice(hz, tau=0.8, m_max=15, eos=11)
    assert list(g["len"]) == list(o["len"]) == [3, 7, 7, -1]
    _check_lattice(g, o, 15)


def test_full_vocabulary_rows():
    svd = require_gpu()
    q, hz = _rows(5, 2, 3, 152064, "bf16", scale=2.0)
    g = host(svd.cps_lattice(q, tau=0.8, m_max=15))
    o = oracle.cps_lattice(hz, tau=0.8, m_max=15)
    _check_lattice(g, o, 15)


@pytest.mark.parametrize("beam,holes", [(1, False), (3, False), (8, False), (3, True)])
def test_beam_matches_oracle_on_the_same_lattice(beam, holes):
    # holes: 5 % of the proxy scores NaN, which rank their expansions last
    svd = require_gpu()
    B, G, M = 12, 10, 6
    q, hz = _rows(7, B, G, 300, "f32", scale=1.0)
    o = oracle.cps_lattice(hz, tau=0.9, m_max=M)
    o["cand_logp"] = o["cand_logp"].astype(np.float32).astype(np.float64)  # the GPU's inputs
    rng = np.random.default_rng(8)
    f = rng.standard_normal((B, G, M, M)).astype(np.float32)
    if holes:
        f[rng.random(f.shape) < 0.05] = np.nan
    ob = oracle.cps_beam(o, f, lam=0.7, beam=beam)
    lat = {k: torch.from_numpy(np.ascontiguousarray(v if k != "cand_logp" else v.astype(np.float32))).cuda()
           for k, v in o.items() if k in ("cand", "cand_logp", "n_cand", "len")}
    g = host(svd.cps_beam(lat, torch.from_numpy(f).cuda(), lam=0.7, beam=beam))
    for b in range(B):
        if ob["rank_margin"][b] < 1e-9:
            continue
        assert np.array_equal(g["paths"][b], ob["paths"][b]), b
        assert np.array_equal(g["path_len"][b], ob["path_len"][b])
        live = ob["path_len"][b] > 0
        assert np.allclose(g["score"][b][live], ob["score"][b][live], atol=1e-4)


def test_lattice_then_beam_end_to_end():
    svd = require_gpu()
    B, G, V, M = 8, 12, 5000, 15
    q, hz = _rows(9, B, G, V, "bf16", scale=1.5, eos=3, eos_at=[(1, 7)])
    f = (np.random.default_rng(2).standard_normal((B, G, M, M)) * 0.3).astype(np.float32)
    gl = svd.cps_lattice(q, tau=0.8, m_max=M, eos=3)
    g = host(svd.cps_beam(gl, torch.from_numpy(f).cuda(), lam=0.5, beam=3))
    ol = oracle.cps_lattice(hz, tau=0.8, m_max=M, eos=3)
    ob = oracle.cps_beam(ol, f, lam=0.5, beam=3)
    compared = 0
    for b in range(B):
        if np.min(ol["cum_margin"][b]) < CUM_EPS or ob["rank_margin"][b] < RANK_EPS:
            continue
        compared += 1
        assert np.array_equal(g["paths"][b], ob["paths"][b]), b
        assert np.allclose(g["score"][b], ob["score"][b], atol=1e-3)
    assert compared >= B - 2
    assert g["path_len"][1, 0] == 8 and g["paths"][1, 0, 7] == 3  # stopped at the EOS


def test_beam_rejects_unusable_inputs():
    svd = require_gpu()
    B, G, M = 3, 4, 4
    lat = {"cand": torch.zeros((B, G, M), dtype=torch.int32, device="cuda"),
           "cand_logp": torch.zeros((B, G, M), dtype=torch.float32, device="cuda"),
           "n_cand": torch.tensor([[1, 2, 1, 1], [1, 5, 1, 1], [1, 1, 1, 1]], dtype=torch.int32,
                                  device="cuda"),
           "len": torch.tensor([4, 4, 9], dtype=torch.int32, device="cuda")}
    g = host(svd.cps_beam(lat, None, beam=2))
    assert list(g["path_len"][:, 0]) == [4, 0, 0]  # n_cand 5 > m_max, len 9 > G
    assert np.all(g["paths"][1:] == -1)
    assert svd.svd_cps_beam(lat["cand"], lat["cand_logp"], lat["n_cand"], lat["len"], None, 1.0,
                            B, 2000, M, 2, lat["cand"], lat["cand_logp"], lat["n_cand"],
                            None) == svd.SVD_EINVAL


def test_lattice_with_many_ties_at_the_top():
    # more tokens tie at the threshold than the candidate list holds: the
    # per-thread sorted lists take over; the lowest indices win the tie
    svd = require_gpu()
    q, hz = _rows(11, 2, 3, 3000, "f32")
    hz = hz.copy()
    hz[0, :, 100:700] = 9.0
    hz[1, 1, ::2] = 7.0
    q = torch.from_numpy(hz).cuda()
    g = host(svd.cps_lattice(q, tau=0.99, m_max=16))
    o = oracle.cps_lattice(hz, tau=0.99, m_max=16)
    _check_lattice(g, o, 16)
    assert list(g["cand"][0, 0, :3]) == [100, 101, 102]


def test_split_rows_with_ties_inside_one_slice():
    # few rows: each row is cut into slices; 600 tied tokens fill one slice's
    # candidate list, whose sorted per-thread lists take over
    svd = require_gpu()
    q, hz = _rows(13, 1, 2, 40000, "f32")
    hz = hz.copy()
    hz[0, 0, 5000:5600] = 9.0
    q = torch.from_numpy(hz).cuda()
    g = host(svd.cps_lattice(q, tau=0.99, m_max=16))
    o = oracle.cps_lattice(hz, tau=0.99, m_max=16)
    _check_lattice(g, o, 16)
    assert list(g["cand"][0, 0, :2]) == [5000, 5001]


# Whole rows held in registers: launches of at least 128 rows of bf16 with at
# most 19 16-byte vectors per thread of a 1024-thread workgroup (V <= 155648);
# V = 155656 is the first size that streams instead.
@pytest.mark.parametrize("V", [152064, 155648, 155656, 8192, 1000])
def test_register_rows_match_oracle(V):
    svd = require_gpu()
    B, G = 16, 8  # 128 rows: whole-row workgroups
    say("register rows", V)
    q, hz = _rows(17 + V % 97, B, G, V, "bf16", scale=2.0)
    g = host(svd.cps_lattice(q, temp_q=0.7, tau=0.8, m_max=15))
    o = oracle.cps_lattice(hz, temp_q=0.7, tau=0.8, m_max=15)
    assert _check_lattice(g, o, 15) <= 2


def test_register_rows_with_ties_infinities_and_nan():
    # in whole-row workgroups held in registers: equal top logits across
    # threads and inside one vector, more ties at the bound than the candidate
    # list holds, rows whose first threads see only -inf, a row of -inf but
    # for a few tokens, and NaN rows (invalid), against the oracle
    svd = require_gpu()
    B, G, V = 16, 8, 152064
    q, hz = _rows(29, B, G, V, "bf16", scale=2.0)
    hz = hz.copy()
    ninf, nan = np.uint16(0xFF80), np.uint16(0x7FC0)
    top = np.uint16(0x4180)  # 16.0
    hz[0, 0, [5, 6, 7, 8000, 151000]] = top              # ties inside one vector and across threads
    hz[0, 1, 1000:1700] = np.uint16(0x4140)              # 700 tokens at 12.0: the list overflows
    hz[1, 0, : V // 2] = ninf                            # the first half of the row is -inf
    # threads 0..511 of the workgroup hold vectors t + 1024 r: all -inf here
    hz[1, 2, ((np.arange(V) // 8) % 1024) < 512] = ninf
    hz[1, 1, :] = ninf                                   # all -inf but four tokens
    hz[1, 1, [3, 70000, 150000, 152063]] = np.uint16(0x3F80)
    hz[2, 3, 123456] = nan                               # NaN: the row is invalid
    hz[3, :, 0:8] = top                                  # a whole vector tied at the top
    q = torch.from_numpy(hz.view(np.int16).copy()).view(torch.bfloat16).cuda()
    g = host(svd.cps_lattice(q, temp_q=1.0, tau=0.9, m_max=16))
    o = oracle.cps_lattice(hz, temp_q=1.0, tau=0.9, m_max=16)
    assert g["len"][2] == o["len"][2] == -1
    _check_lattice(g, o, 16)
    assert list(g["cand"][0, 0, :5]) == [5, 6, 7, 8000, 151000]
    assert list(g["cand"][1, 1, :4]) == [3, 70000, 150000, 152063]


def test_register_rows_bound_from_the_first_vectors():
    # the register form takes its bound from each thread's first vectors
    # (tokens [0, 81920) at V = 152064 with 1024 threads): rows whose best
    # tokens all lie beyond that part, so the bound is loose, with a few
    # hundred tokens at or above it, or so many that the list overflows into
    # the streamed merge; and +0 tied with -0 at the top (equal probabilities:
    # the lower index first), against the oracle
    svd = require_gpu()
    B, G, V = 16, 8, 152064
    first = 10 * 1024 * 8
    rng = np.random.default_rng(41)
    z = (rng.standard_normal((B, G, V)) * 2.0).astype(np.float32)
    z[0, 0, :first] = -8.0                   # every first-part maximum ties at -8: overflow
    z[0, 1, :first] -= 1.5                   # a loose bound: some hundreds listed
    z[0, 2, :first] -= 40.0                  # the first part far below the rest
    z[1, 0, :] = -np.inf                     # +0 and -0 at the top, then -1
    z[1, 0, [3, 50]] = 0.0
    z[1, 0, [100, 90000]] = -0.0
    z[1, 0, [7, 120000, 151999]] = -1.0
    t = torch.from_numpy(z).to(torch.bfloat16)
    hz = t.view(torch.int16).numpy().view(np.uint16).copy()
    assert hz[1, 0, 100] == 0x8000 and hz[1, 0, 50] == 0x0000
    q = t.cuda()
    g = host(svd.cps_lattice(q, temp_q=1.0, tau=0.99, m_max=16))
    o = oracle.cps_lattice(hz, temp_q=1.0, tau=0.99, m_max=16)
    _check_lattice(g, o, 16)
    assert list(g["cand"][1, 0, :7]) == [3, 50, 100, 90000, 7, 120000, 151999]
    # the best tokens of the rows with a low first part lie beyond it
    for j in (0, 1, 2):
        n = int(g["n_cand"][0, j])
        assert n >= 1 and np.all(g["cand"][0, j, :n] >= first), (j, g["cand"][0, j, :n])


def _bf16_rows(z):
    t = torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)).to(torch.bfloat16)
    return t.cuda(), t.view(torch.int16).numpy().view(np.uint16).copy()


def test_register_rows_rising_maxima_and_large_logits():
    # whole rows held in registers whose running maxima rise at every vector
    # (each sum rescaled every time), fall from the first vector on, or tie by
    # the hundred in bf16; and logits near 5000 at temperature 20 (32 apart in
    # bf16, 2.3 octaves), a spread distribution far from zero
    svd = require_gpu()
    B, G, V = 16, 8, 152064
    rng = np.random.default_rng(43)
    ramp = np.arange(V, dtype=np.float32) * 1e-3
    z = (rng.standard_normal((B, G, V)) * 2.0).astype(np.float32)
    z[0, 0] = ramp + rng.standard_normal(V).astype(np.float32)
    z[0, 1] = ramp[::-1] + rng.standard_normal(V).astype(np.float32)
    z[0, 2] = ramp * 5.0  # ties in bf16: hundreds of tokens share each top value
    q, hz = _bf16_rows(z)
    g = host(svd.cps_lattice(q, temp_q=1.0, tau=0.9, m_max=16))
    o = oracle.cps_lattice(hz, temp_q=1.0, tau=0.9, m_max=16)
    assert _check_lattice(g, o, 16) <= 2
    assert g["cand"][0, 0, 0] > V - 8192 and g["cand"][0, 1, 0] < 8192
    z = 5000.0 + rng.standard_normal((B, G, V)).astype(np.float32) * 200.0
    q, hz = _bf16_rows(z)
    g = host(svd.cps_lattice(q, temp_q=20.0, tau=0.8, m_max=15))
    o = oracle.cps_lattice(hz, temp_q=20.0, tau=0.8, m_max=15)
    assert _check_lattice(g, o, 15) <= 2
    assert np.mean(g["n_cand"]) > 2  # a spread distribution, not one token


@pytest.mark.parametrize("temp", [1e-6, 1e-9])
def test_register_rows_at_extreme_temperatures(temp):
    # temperatures of 1e-6 and 1e-9: scaled logits z / temp * log2(e) near
    # 1e7 and past 1e9, so each row's distribution sits on its top token (or
    # its ties), with a row of logits below 0.009 and one with a lone 13.0
    svd = require_gpu()
    B, G, V = 16, 8, 152064
    rng = np.random.default_rng(47)
    z = (rng.standard_normal((B, G, V)) * 2.0).astype(np.float32)
    z[0, 0] = rng.standard_normal(V).astype(np.float32) * 0.002
    z[1, 1, 77] = 13.0  # a row past 11.6
    q, hz = _bf16_rows(z)
    g = host(svd.cps_lattice(q, temp_q=temp, tau=0.8, m_max=15))
    o = oracle.cps_lattice(hz, temp_q=temp, tau=0.8, m_max=15)
    assert _check_lattice(g, o, 15) <= 2
    assert g["cand"][1, 1, 0] == 77


def test_cps_on_the_shared_marginal_workload():
    # the benchmark's search at full size: the 256 shared drafter rows of the
    # shared-marginal workload (B = 16, gamma = 16, V = 152064, bf16), held in
    # registers by the lattice; tau 0.8, M_max 15, beam 3 over random
    # transition scores; every row and every prefix against the oracle
    import workloads as W
    svd = require_gpu()
    cfg = W.get_config("shared_marginal")
    B, G, V, M = cfg.B, cfg.gamma, cfg.V, 15
    d = W.generate_pooled(cfg, device=torch.device("cuda:0"))
    q = d["q_pool"].view(B, G, V)
    assert q.dtype == torch.bfloat16 and q.is_contiguous()
    hz = q.cpu().view(torch.int16).numpy().view(np.uint16)
    f = (np.random.default_rng(cfg.data_seed + 5).standard_normal((B, G, M, M)) * 0.3).astype(
        np.float32)
    gl = svd.cps_lattice(q, temp_q=cfg.temp, tau=0.8, m_max=M)
    g = host(svd.cps_beam(gl, torch.from_numpy(f).cuda(), lam=0.5, beam=3))
    ol = oracle.cps_lattice(hz, temp_q=cfg.temp, tau=0.8, m_max=M)
    flagged = _check_lattice(host(gl), ol, M)
    ob = oracle.cps_beam(ol, f, lam=0.5, beam=3)
    compared = 0
    for b in range(B):
        if np.min(ol["cum_margin"][b]) < CUM_EPS or ob["rank_margin"][b] < RANK_EPS:
            continue
        compared += 1
        assert np.array_equal(g["paths"][b], ob["paths"][b]), b
        assert np.allclose(g["score"][b], ob["score"][b], atol=1e-3)
    say("rows with a cut near tau", flagged, "prefixes compared", compared, "of", B)
    assert compared >= B - 2
