"""The entry points under HIP graph capture.  A call allocates nothing, syncs
nothing and clears its counters and flags with kernels (no memset nodes), so a
serving loop can capture it once and replay it.  Each case captures one call
with a caller-owned workspace, then replays the graph three times with eager
calls of other seeds on the same workspace in between; every replay must give
the eager call's outputs bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import host, require_gpu, say

pytestmark = pytest.mark.gpu

OUT_KEYS = ("selected", "accept_len", "next_token", "scores", "alpha")


def _replays_match(call, other):
    torch.cuda.synchronize()
    ref = host(call())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = call()
    for r in range(3):
        host(other(r))  # eager work on the same workspace between replays
        g.replay()
        torch.cuda.synchronize()
        got = host(out)
        for k in OUT_KEYS:
            if ref.get(k) is None:
                continue
            assert np.array_equal(got[k], ref[k], equal_nan=True), (r, k)
        say("replay", r, "matches the eager call")


@pytest.mark.parametrize("case", [(256, 1, 8, 152064, 0.7), (24, 4, 6, 20000, 1.0)],
                         ids=lambda c: "B%d_K%d_G%d_V%d" % c[:4])
def test_select_and_verify_graph_replays(case):
    svd = require_gpu()
    B, K, G, V, T = case
    cfg = W.Config(70, "custom", B=B, K=K, gamma=G, V=V, dtype="bf16", sigma0=0.75,
                   sigma_step=0.0, temp=T, boost=8.0, boost_prob=1.0)
    d = W.generate(cfg, device="cuda", data_seed=71)
    ws = svd.alloc_workspace(B, K, G, V, d["p"].device)

    def call(seed=5):
        return svd.select_and_verify(d["p"], d["q"], d["drafts"], temp_p=T, seed=seed,
                                     want_alpha=True, want_scores=True, workspace=ws)

    _replays_match(call, lambda r: call(seed=100 + r))


@pytest.mark.parametrize("rule", ["standard", "greedy"])
def test_early_exit_graph_replays(rule):
    # the live list's counters and lists are rebuilt by kernels in every call
    svd = require_gpu()
    B, G, V, T = 300, 12, 20000, 0.9
    cfg = W.Config(72, "custom", B=B, K=1, gamma=G, V=V, dtype="bf16", sigma0=1.2,
                   sigma_step=0.0, temp=T, boost=6.0, boost_prob=1.0)
    d = W.generate(cfg, device="cuda", data_seed=73)
    gb = torch.from_numpy(np.random.default_rng(2).integers(4, G + 1, B).astype(np.int32)).cuda()
    ws = torch.empty(svd.workspace_bytes(B, 1, G, V), dtype=torch.uint8, device="cuda")

    def call(seed=6):
        return svd.verify_window(d["p"], None if rule == "greedy" else d["q"], d["drafts"],
                                 gamma_b=gb, eos=17, rule=rule, early_exit=True, temp_p=T,
                                 seed=seed, want_alpha=True, workspace=ws)

    _replays_match(call, lambda r: call(seed=200 + r))
