"""GPU parity at the full workload sizes (V = 152064, bf16), in the launch
configuration the benchmark times: the whole batch runs on the GPU; the oracle
checks a sample of prefixes one by one; properties that hold at any size are
checked on every prefix; two runs must agree bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import check_ranges, gen, host_inputs, require_gpu, run_select, say
from parity_harness import compare

pytestmark = pytest.mark.gpu

# workload id -> prefixes the oracle recomputes: every prefix of the single
# stream, self-selection and batched-serving batches (2048 positions or fewer),
# the first half of the long window's (16384 of its 32768 positions)
SAMPLES = {2: [0], 3: list(range(16)), 4: list(range(256)), 5: list(range(32))}


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_full_size_workload(orc, cid):
    svd = require_gpu()
    cfg = W.get_config(cid)
    say("workload", cfg.name, "B K gamma V", cfg.B, cfg.K, cfg.gamma, cfg.V)
    d = gen(cfg)
    g = run_select(svd, d, cfg.temp, cfg.seed)
    check_ranges(g, cfg.K, cfg.gamma, cfg.V)
    assert np.all(g["selected"] >= 0)
    # the streak score of the kept draft is the maximum
    kept = g["scores"][np.arange(cfg.B), g["selected"]]
    assert np.all(kept >= g["scores"].max(1))
    # alpha in [0, 1]
    assert np.all((g["alpha"] >= 0) & (g["alpha"] <= 1))
    # run-to-run determinism
    g2 = run_select(svd, d, cfg.temp, cfg.seed)
    for k in ("selected", "accept_len", "next_token", "scores", "alpha"):
        assert np.array_equal(g[k], g2[k]), k
    # oracle on sampled prefixes
    idx = SAMPLES[cid]
    hp, hq, hd = host_inputs(d, idx)
    say("oracle on prefixes", idx)
    rep = compare(orc, hp, hq, hd, g, cfg.temp, cfg.temp, cfg.seed, prefixes=idx)
    say(rep.summary())
    assert rep.ok(), rep.failures
    del hp, hq, hd
    say("mean accepted length %.3f  MAT %.3f" % (g["accept_len"].mean(), g["accept_len"].mean() + 1))
    del d
    torch.cuda.empty_cache()


def test_serving_workload_more_seeds(orc):
    # batched serving: several uniform seeds over the same logits, 16 sampled prefixes each
    svd = require_gpu()
    cfg = W.get_config(4)
    d = gen(cfg)
    idx = list(range(0, 256, 16))
    hp, hq, hd = host_inputs(d, idx)
    for seed in (11, 12, 13):
        # seed 13 without scores: the selection's one-draft path
        g = run_select(svd, d, cfg.temp, seed, row_base=1000, want_scores=seed != 13)
        rep = compare(orc, hp, hq, hd, g, cfg.temp, cfg.temp, seed, row_base=1000, prefixes=idx)
        say(seed, rep.summary())
        assert rep.ok(), rep.failures
