"""Comparison of the HIP library's outputs with the oracle's.

Rules (each follows a reading of the pages where they leave the point open):
  * alpha and beta within ALPHA_TOL absolute; scores within ALPHA_TOL * gamma;
  * selected draft, accepted length and drawn token bit-exact, except where the
    oracle marks the decision as a near-tie:
      - select: the oracle's best and second-best scores differ by less than
        the score tolerance;
      - accept: |u_j - alpha_j| < ACCEPT_EPS at the first position where the
        two accepted lengths part;
      - emit:   t = u * Z lies within EMIT_EPS * Z of a cumulative-weight
        boundary of the drawn token;
  * after an excused mismatch the oracle is re-run with the GPU's decision
    forced, and everything downstream must match exactly again.
Near-tie counts are returned per category with the number of decisions
compared, and the literal 1e-6 CDF-window rate is reported as a statistic.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ALPHA_TOL = 1e-5
ACCEPT_EPS = 1e-5
EMIT_EPS = 1e-10
LITERAL_CDF_WINDOW = 1e-6
EXCUSED_RATE = 1e-4  # excused mismatches per decision kind: under 0.01 %


@dataclass
class ParityReport:
    prefixes: int = 0
    invalid: int = 0
    decisions: dict = field(default_factory=lambda: {"select": 0, "accept": 0, "emit": 0})
    flagged: dict = field(default_factory=lambda: {"select": 0, "accept": 0, "emit": 0})
    near_ties: dict = field(default_factory=lambda: {"select": 0, "accept": 0, "emit": 0})
    literal_cdf_window: int = 0
    max_alpha_err: float = 0.0
    max_beta_err: float = 0.0
    max_score_err: float = 0.0
    failures: list = field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures

    def flag_rate(self) -> float:
        n = sum(self.decisions.values())
        return sum(self.flagged.values()) / max(n, 1)

    def excused_within(self, rate: float = EXCUSED_RATE) -> bool:
        """Excused (near-tie) mismatches at most `rate` of the decisions
        compared, per decision kind (with few decisions: none at all)."""
        return all(self.flagged[k] <= rate * self.decisions[k] for k in self.flagged)

    def merge(self, other: "ParityReport") -> "ParityReport":
        self.prefixes += other.prefixes
        self.invalid += other.invalid
        for k in self.decisions:
            self.decisions[k] += other.decisions[k]
            self.flagged[k] += other.flagged[k]
            self.near_ties[k] += other.near_ties[k]
        self.literal_cdf_window += other.literal_cdf_window
        self.max_alpha_err = max(self.max_alpha_err, other.max_alpha_err)
        self.max_beta_err = max(self.max_beta_err, other.max_beta_err)
        self.max_score_err = max(self.max_score_err, other.max_score_err)
        self.failures += other.failures
        return self

    def summary(self) -> str:
        return ("prefixes=%d invalid=%d decisions=%s mismatches_excused=%s near_ties=%s "
                "literal_cdf_window=%d max_alpha_err=%.3g max_beta_err=%.3g max_score_err=%.3g "
                "failures=%d" % (self.prefixes, self.invalid, self.decisions, self.flagged,
                                 self.near_ties, self.literal_cdf_window, self.max_alpha_err,
                                 self.max_beta_err, self.max_score_err, len(self.failures)))


def _slice(a, b):
    return np.ascontiguousarray(a[b:b + 1])


def _run(orc, greedy, p, q, d, temp_p, temp_q, seed, row_base, want_beta=False, window=None,
         **force):
    """One oracle call in the standard or the greedy-acceptance mode; window: dict of
    gamma_b (aligned with p) and eos for ragged, EOS-aware windows."""
    if window is not None:
        return orc.window_select_and_verify(p, q, d, gamma_b=window.get("gamma_b"),
                                            eos=window.get("eos", -1), greedy=greedy,
                                            temp_p=temp_p, temp_q=temp_q, seed=seed,
                                            row_base=row_base, **force)
    if greedy:
        return orc.greedy_select_and_verify(p, d, temp_p=temp_p, seed=seed, row_base=row_base,
                                            **force)
    return orc.select_and_verify(p, q, d, temp_p=temp_p, temp_q=temp_q, seed=seed,
                                 row_base=row_base, want_beta=want_beta, **force)


def compare(orc, host_p, host_q, host_d, gpu, temp_p, temp_q, seed, row_base=0,
            prefixes=None, rep: ParityReport | None = None, greedy=False,
            window=None) -> ParityReport:
    """host_p/host_q/host_d: host arrays of the prefixes in `prefixes` (in that order);
    gpu: dict of host numpy outputs of the full batch (selected may be None for svd_verify).
    greedy: compare with the oracle's greedy-acceptance mode (host_q is then unused).
    window: ragged, EOS-aware windows: dict(gamma_b aligned with the host arrays, eos).
    """
    rep = rep or ParityReport()
    B, K, G1, V = host_p.shape
    G = G1 - 1
    idx = list(range(B)) if prefixes is None else list(prefixes)
    assert len(idx) == B
    want_beta = gpu.get("beta") is not None
    # uniform rows follow the batch index of each prefix
    rows = np.array(idx, dtype=np.int64)
    res = _oracle_rows(orc, host_p, host_q, host_d, temp_p, temp_q, seed, row_base, rows,
                       want_beta, greedy, window)
    sel_tol = ALPHA_TOL * G
    for i, b in enumerate(idx):
        rep.prefixes += 1
        g_sel = int(gpu["selected"][b]) if gpu.get("selected") is not None else 0
        g_L = int(gpu["accept_len"][b])
        g_tok = int(gpu["next_token"][b])
        o_sel, o_L, o_tok = int(res.selected[i]), int(res.accept_len[i]), int(res.next_token[i])
        if o_sel < 0 or o_L < 0:
            rep.invalid += 1
            if not (g_L == -1 and g_tok == -1 and (gpu.get("selected") is None or g_sel == -1)):
                rep.failures.append((b, "invalid prefix not reported", (g_sel, g_L, g_tok)))
            continue
        if gpu.get("alpha") is not None:
            ga, oa = gpu["alpha"][b].astype(np.float64), res.alpha[i]
            # positions outside a window are NaN on both sides
            if not np.array_equal(np.isnan(ga), np.isnan(oa)):
                rep.failures.append((b, "alpha NaN pattern", (ga, oa)))
            d = np.abs(ga - oa)[~np.isnan(oa)]
            e = float(d.max()) if d.size else 0.0
            rep.max_alpha_err = max(rep.max_alpha_err, e)
            if not e <= ALPHA_TOL:
                rep.failures.append((b, "alpha", e))
        if want_beta:
            e = float(np.max(np.abs(gpu["beta"][b].astype(np.float64) - res.beta[i])))
            rep.max_beta_err = max(rep.max_beta_err, e)
            if not e <= ALPHA_TOL:
                rep.failures.append((b, "beta", e))
        if gpu.get("scores") is not None:
            e = float(np.max(np.abs(gpu["scores"][b].astype(np.float64) - res.scores[i])))
            rep.max_score_err = max(rep.max_score_err, e)
            if not e <= sel_tol:
                rep.failures.append((b, "scores", e))

        pb = _slice(host_p, i)
        qb = None if greedy else _slice(host_q, i)
        db = _slice(host_d, i)
        wb = _window_slice(window, i)
        row = row_base + b
        cur = res
        ci = i
        # 1. selection
        if K > 1:
            rep.decisions["select"] += 1
            if res.select_gap[i] < sel_tol:
                rep.near_ties["select"] += 1
            if g_sel != o_sel:
                if res.select_gap[i] < sel_tol:
                    rep.flagged["select"] += 1
                    cur = _run(orc, greedy, pb, qb, db, temp_p, temp_q, seed, row, window=wb,
                               force_k=np.array([g_sel], np.int32))
                    ci = 0
                else:
                    rep.failures.append((b, "selected", (g_sel, o_sel, res.select_gap[i])))
                    continue
        # 2. accepted length
        o_L = int(cur.accept_len[ci])
        m = cur.accept_margin[ci]
        rep.decisions["accept"] += min(o_L, G - 1) + 1 if o_L < G else G
        rep.near_ties["accept"] += int(np.sum(m[:min(o_L + 1, G)] < ACCEPT_EPS))
        if g_L != o_L:
            j = min(g_L, o_L)
            if 0 <= j < G and m[j] < ACCEPT_EPS:
                rep.flagged["accept"] += 1
                cur = _run(orc, greedy, pb, qb, db, temp_p, temp_q, seed, row, window=wb,
                           force_k=np.array([g_sel], np.int32), force_L=np.array([g_L], np.int32))
                ci = 0
            else:
                rep.failures.append((b, "accept_len", (g_L, o_L, float(m[j]) if 0 <= j < G else None)))
                continue
        # 3. drawn token
        rep.decisions["emit"] += 1
        em = float(cur.emit_margin[ci])
        if em < LITERAL_CDF_WINDOW:
            rep.literal_cdf_window += 1
        if em < EMIT_EPS:
            rep.near_ties["emit"] += 1
        o_tok = int(cur.next_token[ci])
        if g_tok != o_tok:
            if em < EMIT_EPS:
                rep.flagged["emit"] += 1
            else:
                rep.failures.append((b, "next_token", (g_tok, o_tok, em)))
    return rep


def _window_slice(window, i):
    if window is None:
        return None
    gb = window.get("gamma_b")
    return dict(eos=window.get("eos", -1),
                gamma_b=None if gb is None else np.ascontiguousarray(gb[i:i + 1]))


def _oracle_rows(orc, host_p, host_q, host_d, temp_p, temp_q, seed, row_base, rows, want_beta,
                 greedy=False, window=None):
    """Oracle over a host batch whose prefix i sits at batch row rows[i]."""
    rows = np.asarray(rows)
    if len(rows) and np.all(np.diff(rows) == 1):
        return _run(orc, greedy, host_p, host_q, host_d, temp_p, temp_q, seed,
                    row_base + int(rows[0]), want_beta, window)
    parts = [_run(orc, greedy, _slice(host_p, i), None if greedy else _slice(host_q, i),
                  _slice(host_d, i), temp_p, temp_q, seed, row_base + int(r), want_beta,
                  _window_slice(window, i))
             for i, r in enumerate(rows)]
    out = parts[0]
    for f in out.__dataclass_fields__:
        vals = [getattr(pp, f) for pp in parts]
        if vals[0] is not None:
            setattr(out, f, np.concatenate(vals, 0))
    return out
