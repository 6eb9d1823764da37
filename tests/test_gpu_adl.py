"""Adaptive draft length on the GPU (svd_adl_next) against the oracle, bit for
bit: random inputs with every kind of invalid prefix mixed in, and a closed
loop in which each step's windows come from the previous step's controller
output on the device, with the window verification compared with the oracle at
every step."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import gen, host_inputs, require_gpu, say
from parity_harness import compare

pytestmark = pytest.mark.gpu

KW = dict(k_min=2, k_max=40, step=4, shift=2, slack=64)


def test_random_inputs_match_the_oracle(orc):
    svd = require_gpu()
    rng = np.random.default_rng(17)
    for B, K, G, eos in ((20000, 3, 48, 5), (777, 1, 4096, 11), (1, 64, 1, -1)):
        d = rng.integers(0, 40, size=(B, K, G)).astype(np.int32)
        gb = rng.integers(-1, G + 3, size=B).astype(np.int32)
        sel = rng.integers(-1, K, size=B).astype(np.int32)
        L = np.array([rng.integers(-1, max(int(n), 0) + 2) for n in gb], np.int32)
        st = rng.integers(-50, 256 * min(G, 64) + 50, size=(B, 2)).astype(np.int32)
        st[::11] = (1 << 20) + 1
        for kw in (KW, dict(k_min=1, k_max=4096, step=0, shift=0, slack=0),
                   dict(k_min=3, k_max=7, step=4096, shift=16, slack=1 << 20)):
            want_next, want_st = orc.adl_next(d, sel, L, st, gamma_b=gb, eos=eos, **kw)
            dev = {k: torch.from_numpy(v).cuda() for k, v in
                   dict(d=d, sel=sel, L=L, gb=gb, st=st.copy()).items()}
            # host-side checks of what the kernel assumes, before the launch
            assert dev["d"].shape == (B, K, G) and dev["st"].shape == (B, 2)
            got = svd.adl_next(dev["d"], dev["sel"], dev["L"], dev["st"], gamma_b=dev["gb"],
                               eos=eos, **kw)
            torch.cuda.synchronize()
            assert np.array_equal(got.cpu().numpy(), want_next), (B, K, G, kw)
            assert np.array_equal(dev["st"].cpu().numpy(), want_st), (B, K, G, kw)
        say("adl B=%d K=%d gamma=%d: equal" % (B, K, G))


@pytest.mark.parametrize("rule", ["standard", "greedy"])
def test_closed_loop_with_window_verification(orc, rule):
    # 48 prefixes, K = 2 drafts of up to 32 positions over V = 3000; the drafts
    # of a third of the prefixes hold an EOS; six steps, each verifying the
    # windows the previous step's controller chose on the device
    svd = require_gpu()
    cfg = W.Config(91, "custom", B=48, K=2, gamma=32, V=3000, dtype="bf16", sigma0=0.3,
                   sigma_step=0.02, temp=1.0, boost=8.0, boost_prob=1.0)
    d = gen(cfg, data_seed=23)
    eos = 7
    dr = d["drafts"].clone()
    for b in range(0, cfg.B, 3):
        dr[b, :, 5 + (b % 20)] = eos
    d["drafts"] = dr.contiguous()
    hp, hq, hd = host_inputs(d)
    greedy = rule == "greedy"
    kw = dict(KW, k_max=cfg.gamma)  # a window never outgrows the padded arrays
    gb = torch.full((cfg.B,), 4, dtype=torch.int32, device="cuda")
    avg = torch.full((cfg.B, 2), 256 * 4, dtype=torch.int32, device="cuda")
    st_host = avg.cpu().numpy()
    windows = []
    for step in range(6):
        out = svd.verify_window(d["p"], None if greedy else d["q"], d["drafts"], gamma_b=gb,
                                eos=eos, rule=rule, seed=100 + step)
        nxt = svd.adl_next(d["drafts"], out["selected"], out["accept_len"], avg, gamma_b=gb,
                           eos=eos, **kw)
        torch.cuda.synchronize()
        g = {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}
        gbh = gb.cpu().numpy()
        rep = compare(orc, hp, hq, hd, g, 1.0, 1.0, 100 + step, greedy=greedy,
                      window=dict(gamma_b=gbh, eos=eos))
        assert rep.ok(), (step, rep.failures[:3])
        want_next, st_host = orc.adl_next(hd, g["selected"], g["accept_len"], st_host,
                                          gamma_b=gbh, eos=eos, **kw)
        assert np.array_equal(nxt.cpu().numpy(), want_next), step
        assert np.array_equal(avg.cpu().numpy(), st_host), step
        windows.append(want_next)
        gb = nxt
    w = np.array(windows)
    say(rule, "windows per step (mean):", w.mean(1))
    assert np.all((w >= kw["k_min"]) & (w <= cfg.gamma))
