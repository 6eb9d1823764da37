"""Statistics shared by the CPU and GPU distribution checks."""
import numpy as np
from scipy.special import softmax
from scipy.stats import chi2

import workloads as W


def _chisq_p(counts, probs):
    """Chi-square p-value with bins of expected count < 5 merged into one."""
    n = counts.sum()
    exp = probs * n
    big = exp >= 5
    c = list(counts[big]) + ([counts[~big].sum()] if (~big).any() else [])
    e = list(exp[big]) + ([exp[~big].sum()] if (~big).any() else [])
    c, e = np.array(c, float), np.array(e, float)
    m = e > 0
    stat = ((c[m] - e[m]) ** 2 / e[m]).sum()
    return chi2.sf(stat, max(m.sum() - 1, 1))


def tiny_trials(orc, n, chunk=250_000):
    cfg = W.get_config(1)
    base = W.generate(cfg)
    zp, zq = W.to_host(base["p"]), W.to_host(base["q"])
    drafts = W.tiny_trial_drafts(base["q"], n, cfg.temp, seed=cfg.data_seed + 17).numpy()
    L = np.empty(n, np.int32)
    tok = np.empty(n, np.int32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        bp = np.ascontiguousarray(np.broadcast_to(zp, (e - s,) + zp.shape[1:]))
        bq = np.ascontiguousarray(np.broadcast_to(zq, (e - s,) + zq.shape[1:]))
        r = orc.select_and_verify(bp, bq, drafts[s:e], temp_p=cfg.temp, seed=cfg.seed,
                                  row_base=s)
        L[s:e] = r.accept_len
        tok[s:e] = r.next_token
    return cfg, zp, zq, drafts, L, tok


def committed_token_pvalues(zp, zq, drafts, L, tok, temp):
    G = drafts.shape[-1]
    V = zp.shape[-1]
    pv = []
    for j in range(G + 1):
        sel = L >= j
        y = np.where(L[sel] == j, tok[sel], drafts[sel, 0, min(j, G - 1)])
        counts = np.bincount(y, minlength=V)
        pj = softmax(zp[0, 0, j].astype(np.float64) / np.float64(np.float32(temp)))
        pv.append(_chisq_p(counts, pj))
    return pv


def accepted_length_pvalue(zp, zq, L, temp):
    G = zq.shape[2]
    T = np.float64(np.float32(temp))
    beta = np.array([np.minimum(softmax(zp[0, 0, j] / T), softmax(zq[0, 0, j] / T)).sum()
                     for j in range(G)])
    law = np.array([np.prod(beta[:j]) * (1 - beta[j]) for j in range(G)] + [np.prod(beta)])
    return _chisq_p(np.bincount(L, minlength=G + 1), law)
