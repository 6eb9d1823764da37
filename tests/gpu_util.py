"""Helpers of the GPU tests: run the library on device inputs, bring results home."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as W


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import lossless_draft_verification_verifier_amd as svd  # fails loudly without libsvd.so
    return svd


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(out: dict) -> dict:
    return {k: (None if v is None else v.detach().cpu().numpy()) for k, v in out.items()}


def gen(cfg, **kw):
    """Device inputs for a workload (optionally resized)."""
    return W.generate(cfg, device="cuda", **kw)


def host_inputs(d, prefixes=None):
    if prefixes is None:
        return W.to_host(d["p"]), W.to_host(d["q"]), W.to_host(d["drafts"])
    idx = torch.as_tensor(list(prefixes), device=d["p"].device)
    return (W.to_host(d["p"].index_select(0, idx)), W.to_host(d["q"].index_select(0, idx)),
            W.to_host(d["drafts"].index_select(0, idx)))


def run_select(svd, d, temp, seed, row_base=0, want_alpha=True, want_beta=False,
               want_scores=True):
    out = svd.select_and_verify(d["p"], d["q"], d["drafts"], temp_p=temp, seed=seed,
                                row_base=row_base, want_alpha=want_alpha, want_beta=want_beta,
                                want_scores=want_scores)
    torch.cuda.synchronize()
    return host(out)


def check_ranges(g, K, G, V):
    sel, L, tok = g["selected"], g["accept_len"], g["next_token"]
    ok = sel >= 0
    assert np.all((sel[ok] < K) & (L[ok] >= 0) & (L[ok] <= G) & (tok[ok] >= 0) & (tok[ok] < V))
    assert np.all((L[~ok] == -1) & (tok[~ok] == -1))
