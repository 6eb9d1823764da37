"""Calls every C entry point of a libsvd build with arguments its host-side
checks reject (fake, never dereferenced addresses: no HIP call is reached),
including dtype and rule values outside the enumerators, and prints the status
codes.  Run by tests/test_abi_sanitized.py against a build whose host code has
AddressSanitizer and UBSan, and against the product library."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import lossless_draft_verification_verifier_amd as svd  # noqa: E402

L = svd.Library(sys.argv[1])
P, Q, D, S, AL, T, WS = 4096, 8192, 12288, 16384, 20480, 24576, 1 << 20
out = []


def sv(**kw):
    a = dict(p=P, q=Q, d=D, dtype=svd.SVD_BF16, B=2, K=2, G=3, V=100, tp=1.0, tq=1.0, sel=S,
             L=AL, tok=T, ws=WS, n=0)
    a.update(kw)
    return L.svd_select_and_verify(a["p"], a["q"], a["d"], a["dtype"], a["B"], a["K"], a["G"],
                                   a["V"], a["tp"], a["tq"], 0, 0, a["sel"], a["L"], a["tok"],
                                   None, None, None, a["ws"], a["n"], None)


for kw in (dict(p=None), dict(dtype=2), dict(dtype=-5), dict(dtype=0x7FFFFFFF), dict(B=0),
           dict(B=1 << 40), dict(K=0), dict(K=65), dict(G=0), dict(G=4097), dict(V=0),
           dict(V=-3), dict(tp=0.0), dict(tq=float("nan")), dict(tp=1e-40), dict(tp=4.5e-39),
           dict(ws=WS + 64), dict()):
    out.append(sv(**kw))
out.append(L.svd_verify(P, Q, None, svd.SVD_BF16, 1, 2, 10, 1.0, 1.0, 0, 0, S, AL, None, None,
                        WS, 0, None))
out.append(L.svd_verify(P, Q, D, 9, 1, 2, 10, 1.0, 1.0, 0, 0, S, AL, None, None, WS, 0, None))
for dt, tp in ((svd.SVD_BF16, 0.0), (3, 1.0), (svd.SVD_F32, float("inf"))):
    out.append(L.svd_greedy_select_and_verify(P, D, dt, 2, 2, 3, 100, tp, 0, 0, S, AL, T, None,
                                              None, WS, 0, None))
    out.append(L.svd_greedy_verify(P, D, dt, 1, 2, 10, tp, 0, 0, S, AL, None, WS, 0, None))
for rule in (2, -1, svd.SVD_RULE_STANDARD):
    out.append(L.svd_select_and_verify_rows(rule, P, 10, D, Q, 0, D, D, svd.SVD_BF16, 2, 2, 3,
                                            100, 1.0, 1.0, 0, 0, S, AL, T, None, None, WS, 0,
                                            None))
    out.append(L.svd_verify_window(rule, P, Q, D, None, -1, 1, svd.SVD_BF16, 2, 1, 3, 100, 1.0,
                                   1.0, 0, 0, S, AL, T, None, None, WS, 0, None))
for kw in (dict(dtype=2), dict(tau=0.0), dict(m=17), dict(eos=100), dict(V=0)):
    a = dict(dtype=svd.SVD_BF16, tau=0.8, m=15, eos=-1, V=100)
    a.update(kw)
    out.append(L.svd_cps_lattice(Q, a["dtype"], 2, 4, a["V"], 1.0, a["tau"], a["m"], a["eos"],
                                 D, S, AL, T, WS, 0, None))
for kw in (dict(beam=0), dict(beam=9), dict(G=1025), dict(m=0)):
    a = dict(beam=3, G=4, m=15)
    a.update(kw)
    out.append(L.svd_cps_beam(D, S, AL, T, None, 1.0, 2, a["G"], a["m"], a["beam"], P, Q, D,
                              None))
for kw in (dict(B=0), dict(k_min=0), dict(step=-1), dict(shift=17), dict(slack=-1)):
    a = dict(B=4, k_min=1, step=4, shift=2, slack=64)
    a.update(kw)
    out.append(L.svd_adl_next(D, S, AL, None, -1, a["B"], 2, 8, a["k_min"], 16, a["step"],
                              a["shift"], a["slack"], T, P, None))
out.append(L.svd_select_and_verify_noalloc(P, Q, D, svd.SVD_BF16, 2048, 1, 8, 152064, 1.0, 1.0,
                                           0, 0, S, AL, T, None, None, None, None))
out.append(L.svd_select_and_verify_noalloc(P, Q, D, 5, 2, 1, 8, 100, 1.0, 1.0, 0, 0, S, AL, T,
                                           None, None, None, None))
for args in ((256, 1, 8, 152064), (1 << 40, 1, 1, 1), (1, 65, 1, 1), (-1, 1, 1, 1)):
    out.append(L.svd_workspace_bytes(*args))
out.append(L.svd_rows_workspace_bytes(2, 2, 3, 100, 0, 10))
out.append(L.svd_cps_workspace_bytes(2, 4))
out += [L.svd_strerror(c) for c in (0, -1, -2, -3, -4, -5, 12345, -(1 << 31))]
print(out)
