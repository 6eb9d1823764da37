"""GPU parity on small and ragged shapes: every output of every prefix against
the oracle, under the rules of parity_harness (several tiles of the row loop,
ragged vocabulary tails, unaligned rows on the element-wise path, K up to 64,
gamma beyond one wave of 64)."""
import numpy as np
import pytest

import workloads as W
from gpu_util import gen, host_inputs, require_gpu, run_select, say, check_ranges
from parity_harness import compare

pytestmark = pytest.mark.gpu

BASE = W.get_config(3)

CASES = [
    # (B, K, gamma, V, dtype, temp)
    (1, 1, 4, 32, "f32", 1.0),
    (3, 1, 5, 1000, "bf16", 1.0),        # 16-byte rows, vector path, ragged last tile
    (3, 2, 3, 1001, "bf16", 0.7),        # odd V: element-wise path
    (2, 3, 7, 4099, "f32", 1.3),         # odd V, fp32
    (5, 4, 6, 8192, "bf16", 0.7),        # exactly one draw segment
    (4, 3, 5, 8193, "bf16", 1.0),        # one token into a second segment
    (2, 8, 16, 20000, "bf16", 1.0),
    (3, 1, 70, 2048, "bf16", 1.0),       # gamma beyond one wave of 64
    (1, 64, 2, 512, "bf16", 2.0),        # K at its limit
    (2, 2, 4096, 64, "f32", 1.0),        # gamma at its limit
    (17, 2, 4, 3000, "f32", 0.5),
    (800, 1, 2, 8193, "bf16", 1.0),      # a batch drawn in segments of 8192: one-token second segment
    (3, 2, 4, 1032, "bf16", 1.0),        # segments of 1024: an 8-token second segment
    (2, 1, 3, 70008, "bf16", 0.7),       # 69 segments of 1024: runs of segments per lane in the pick
    (2, 1, 1, 1, "f32", 1.0),            # V = 1: every row is one token
    (3, 2, 2, 2, "bf16", 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_K%d_G%d_V%d_%s" % c[:5])
@pytest.mark.parametrize("seed", [1, 20261202])
def test_small_shapes_match_oracle(orc, case, seed):
    svd = require_gpu()
    B, K, G, V, dt, T = case
    say("case", case, "seed", seed)
    cfg = W.Config(99, "custom", B=B, K=K, gamma=G, V=V, dtype=dt, sigma0=1.0, sigma_step=0.02,
                   temp=T, boost=6.0, boost_prob=0.8)
    d = gen(cfg, data_seed=seed * 7 + V)
    g = run_select(svd, d, T, seed, row_base=seed % 5, want_beta=True)
    check_ranges(g, K, G, V)
    hp, hq, hd = host_inputs(d)
    rep = compare(orc, hp, hq, hd, g, T, T, seed, row_base=seed % 5)
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]
    assert rep.invalid == 0


@pytest.mark.parametrize("temp", [0.05, 0.2, 8.0, 40.0])
def test_extreme_temperatures(orc, temp):
    # 0.05: nearly one-hot rows, draw weights down to 2^-500 and below the
    # exp's underflow clamp; 40: nearly uniform rows, p and q close, so the
    # residual is small and most tokens sit near the p > q margin
    svd = require_gpu()
    B, K, G, V = 6, 2, 5, 9000
    say("temp", temp)
    cfg = W.Config(99, "custom", B=B, K=K, gamma=G, V=V, dtype="bf16", sigma0=0.5,
                   sigma_step=0.05, temp=temp, boost=6.0, boost_prob=0.8)
    d = gen(cfg, data_seed=int(temp * 100) + 3)
    g = run_select(svd, d, temp, 9, want_beta=True)
    check_ranges(g, K, G, V)
    hp, hq, hd = host_inputs(d)
    rep = compare(orc, hp, hq, hd, g, temp, temp, 9)
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]
    assert rep.invalid == 0


@pytest.mark.parametrize("seed", range(8))
def test_tiny_workload_matches_oracle(orc, seed):
    svd = require_gpu()
    cfg = W.get_config(1)
    d = gen(cfg)
    g = run_select(svd, d, cfg.temp, seed)
    rep = compare(orc, *host_inputs(d), g, cfg.temp, cfg.temp, seed)
    assert rep.ok(), rep.failures


def test_distinct_temperatures(orc):
    svd = require_gpu()
    cfg = W.Config(98, "custom", B=4, K=3, gamma=5, V=3000, dtype="bf16", sigma0=1.0,
                   sigma_step=0.0, temp=1.0, boost=6.0, boost_prob=1.0)
    d = gen(cfg, data_seed=5)
    import torch
    out = svd.select_and_verify(d["p"], d["q"], d["drafts"], temp_p=0.8, temp_q=1.7, seed=3,
                                want_alpha=True, want_scores=True)
    torch.cuda.synchronize()
    g = {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}
    rep = compare(orc, *host_inputs(d), g, 0.8, 1.7, 3)
    assert rep.ok(), rep.failures


def test_many_prefixes_flag_rates(orc):
    # 400 prefixes of a mid-size vocabulary: no unflagged mismatch, few near-ties
    svd = require_gpu()
    cfg = W.Config(97, "custom", B=400, K=2, gamma=8, V=6000, dtype="bf16", sigma0=0.75,
                   sigma_step=0.0, temp=0.7, boost=8.0, boost_prob=1.0)
    d = gen(cfg, data_seed=11)
    g = run_select(svd, d, 0.7, 9)
    rep = compare(orc, *host_inputs(d), g, 0.7, 0.7, 9)
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]
    assert rep.excused_within(), rep.summary()


# 8 prefixes of 20000 tokens are drawn in segments of 1024 tokens, 400 in
# segments of 8192 (the draw cuts rows finer when a batch is small)
MARGIN_BATCHES = [8, 400]


def _margin_case(B, seed):
    # q equals p except at the drafted token (a median one), raised by 2, so
    # most drafts are rejected at position 0 and S_q / S_p is within the
    # classification margin of 1
    import torch
    G, V = 3, 20000
    gen_ = torch.Generator(device="cuda").manual_seed(seed)
    zp = torch.randn((B, 1, G + 1, V), generator=gen_, device="cuda") * 2.0
    zq = zp[:, :, :G].clone()
    x = torch.argsort(zp[:, :, :G], dim=-1)[..., V // 2].to(torch.int32)
    zq.scatter_add_(-1, x.long().unsqueeze(-1), torch.full((B, 1, G, 1), 2.0, device="cuda"))
    return G, {"p": zp.contiguous(), "q": zq.contiguous(), "drafts": x.contiguous()}


@pytest.mark.parametrize("B", MARGIN_BATCHES)
def test_residual_inside_the_margin_everywhere(orc, B):
    # at one temperature every other token has w_p == w_q exactly: the margin
    # tokens settle as one sum whose sign is that of 1/S_p - 1/S_q
    svd = require_gpu()
    G, d = _margin_case(B, 77)
    g = run_select(svd, d, 1.0, 5)
    say("accept lengths", g["accept_len"])
    assert (g["accept_len"] < G).sum() >= B // 2
    rep = compare(orc, *host_inputs(d), g, 1.0, 1.0, 5)
    say(rep.summary())
    assert rep.ok(), rep.failures


@pytest.mark.parametrize("shift", [1e-3, -1e-2])
def test_equal_logit_class_with_distinct_maxima(orc, shift):
    # the case above with q's maximum logit also moved by a small shift: the
    # tokens of equal logits share one ratio exp(M_q - M_p) S_q / S_p != 1,
    # inside the margin, and settle as one class of that ratio's sign
    svd = require_gpu()
    import torch
    G, d = _margin_case(40, 79)
    q = d["q"]
    top = torch.argmax(q, dim=-1, keepdim=True)
    q.scatter_add_(-1, top, torch.full(top.shape, shift, device="cuda"))
    g = run_select(svd, d, 1.0, 7)
    say("accept lengths", g["accept_len"])
    assert (g["accept_len"] < G).sum() >= 20
    rep = compare(orc, *host_inputs(d), g, 1.0, 1.0, 7)
    say(rep.summary())
    assert rep.ok(), rep.failures


@pytest.mark.parametrize("B", MARGIN_BATCHES)
def test_margin_classes_of_one_logit_difference(orc, B):
    # the case above with 2 % of q's logits lowered by 2^-14 and 1 % by 2^-13:
    # each difference is one class of about 60-160 margin tokens per segment,
    # more than a segment keeps singly, merged class by class
    svd = require_gpu()
    import torch
    G, d = _margin_case(B, 80)
    q = d["q"]
    g_ = torch.Generator(device="cuda").manual_seed(81)
    u = torch.rand(q.shape, generator=g_, device="cuda")
    q.sub_(torch.where(u < 0.02, 2.0 ** -14, torch.where(u < 0.03, 2.0 ** -13, 0.0)))
    g = run_select(svd, d, 1.0, 8)
    say("accept lengths", g["accept_len"])
    assert (g["accept_len"] < G).sum() >= B // 2
    rep = compare(orc, *host_inputs(d), g, 1.0, 1.0, 8)
    say(rep.summary())
    assert rep.ok(), rep.failures


@pytest.mark.parametrize("B", MARGIN_BATCHES)
def test_residual_margin_lists_overflow(orc, B):
    # the same rows with q read at a temperature 2^-17 above p's: every p/q ratio
    # is within the margin and almost none is exactly 1, so every segment's
    # list of uncertain tokens overflows and the pick recomputes its mass exactly
    svd = require_gpu()
    import torch
    G, d = _margin_case(B, 78)
    tq = 1.0 + 2.0 ** -17
    out = svd.select_and_verify(d["p"], d["q"], d["drafts"], temp_p=1.0, temp_q=tq, seed=6,
                                want_alpha=True, want_scores=True)
    torch.cuda.synchronize()
    g = {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}
    say("accept lengths", g["accept_len"])
    assert (g["accept_len"] < G).sum() >= B // 2
    rep = compare(orc, *host_inputs(d), g, 1.0, tq, 6)
    say(rep.summary())
    assert rep.ok(), rep.failures


@pytest.mark.parametrize("V", [5000, 20000, 40001])
def test_bonus_draws_across_segments(orc, V):
    svd = require_gpu()
    cfg = W.Config(92, "custom", B=6, K=2, gamma=3, V=V, dtype="bf16", sigma0=1.0,
                   sigma_step=0.0, temp=0.9, boost=6.0, boost_prob=0.5)
    d = gen(cfg, data_seed=V)
    d["q"].copy_(d["p"][:, :, :3])  # alpha == 1: every prefix draws its bonus token
    for seed in (1, 2):
        g = run_select(svd, d, 0.9, seed)
        assert np.all(g["accept_len"] == 3)
        rep = compare(orc, *host_inputs(d), g, 0.9, 0.9, seed)
        assert rep.ok(), rep.failures


@pytest.mark.parametrize("temp", [1.0, 0.7])
def test_large_batch_edge_logits(orc, temp):
    # 512 prefixes over rows with -inf (masked tokens), near-zero and large
    # logit magnitudes, a ragged last draw segment; the oracle checks a sample
    # of prefixes
    svd = require_gpu()
    import torch
    B, G, V = 512, 2, 3 * 8192 + 5
    g_ = torch.Generator(device="cuda").manual_seed(90)
    zp = torch.randn((B, 1, G + 1, V), generator=g_, device="cuda") * 2.0
    u = torch.rand((B, 1, G + 1, V), generator=g_, device="cuda")
    zp = torch.where(u < 0.01, torch.full_like(zp, float("-inf")), zp)
    zp = torch.where((u >= 0.01) & (u < 0.02), zp * 1e-5, zp)
    zp = torch.where((u >= 0.02) & (u < 0.021), zp * 25.0, zp)
    zq = zp[:, :, :G] + 0.75 * torch.randn((B, 1, G, V), generator=g_, device="cuda")
    zp, zq = zp.to(torch.bfloat16), zq.to(torch.bfloat16)
    gum = -torch.log(-torch.log(torch.rand((B, 1, G, V), generator=g_, device="cuda")))
    x = torch.argmax(zq.float() / temp + gum, dim=-1).to(torch.int32)
    d = {"p": zp.contiguous(), "q": zq.contiguous(), "drafts": x.contiguous()}
    g = run_select(svd, d, temp, 12)
    idx = list(range(0, B, 16))
    hp, hq, hd = host_inputs(d, idx)
    rep = compare(orc, hp, hq, hd, g, temp, temp, 12, prefixes=idx)
    say(rep.summary())
    assert rep.ok(), rep.failures
    assert rep.invalid == 0


@pytest.mark.parametrize("B,V", [(2, 300000), (30, 2_200_000)])
@pytest.mark.parametrize("bonus", [False, True])
def test_more_draw_segments_than_the_pick_stages(orc, B, V, bonus):
    # more than 256 draw segments per row (2 prefixes of 300000 tokens in
    # segments of 1024: 293; 30 of 2.2M in segments of 8192: 269): the pick
    # reads the segment records and keeps the masses in global memory and
    # scans runs of five segments per lane; bonus: q = p, every prefix draws
    # from its bonus row
    svd = require_gpu()
    say("segments", B, V, "bonus", bonus)
    cfg = W.Config(91, "custom", B=B, K=1, gamma=3, V=V, dtype="bf16", sigma0=1.0,
                   sigma_step=0.0, temp=0.9, boost=8.0, boost_prob=1.0)
    d = gen(cfg, data_seed=V + B)
    if bonus:
        d["q"].copy_(d["p"][:, :, :3])
    g = run_select(svd, d, 0.9, 4)
    check_ranges(g, 1, 3, V)
    if bonus:
        assert np.all(g["accept_len"] == 3)
    rep = compare(orc, *host_inputs(d), g, 0.9, 0.9, 4)
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]
    assert rep.invalid == 0
