"""Seeded synthetic logits and drafts.

Recipe (per prefix b, with its own generator seeded from (data_seed, b)):
  * verifier logits z_p ~ N(0, 2^2), i.i.d. over the vocabulary, for all K
    drafts and gamma+1 rows; every row gets a mode token m ~ U{0..V-1} whose
    logit is raised by `boost` (on a `boost_prob` share of rows);
  * row 0 of p is shared by the K drafts of a prefix: all drafts start from the
    same prefix s, so the verifier's first posterior is the same;
  * drafter logits z_q = z_p + sigma_j * N(0, 1) for rows j < gamma, independent
    per draft and row;
  * bf16 workloads round the fp32 values to nearest-even;
  * drafted tokens x_j are sampled from softmax(z_q_j / T) of the rounded logits
    with the Gumbel-max trick: argmax_v (z_q_jv / T + G_v), G_v i.i.d. Gumbel.

Nothing here evaluates the verification rule; the draft sampler stands in for
the diffusion drafter.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import Config


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed & 0x7FFFFFFFFFFFFFFF)
    return g


def _gumbel_argmax(z: torch.Tensor, temp: float, g: torch.Generator) -> torch.Tensor:
    u = torch.rand(z.shape, generator=g, device=z.device, dtype=torch.float32)
    gumbel = -torch.log(-torch.log(u))
    return torch.argmax(z.float() / temp + gumbel, dim=-1).to(torch.int32)


def _one_prefix(cfg: Config, b: int, data_seed: int, device, K: int, G: int, V: int,
                tdtype: torch.dtype):
    g = _gen(device, data_seed * 1_000_003 + b)
    zp = torch.randn((K, G + 1, V), generator=g, device=device, dtype=torch.float32) * 2.0
    mode = torch.randint(0, V, (K, G + 1, 1), generator=g, device=device)
    hit = torch.rand((K, G + 1, 1), generator=g, device=device) < cfg.boost_prob
    zp.scatter_add_(-1, mode, hit.float() * cfg.boost)
    zp[1:, 0, :] = zp[0, 0, :]
    sig = cfg.sigma0 + cfg.sigma_step * torch.arange(G, device=device, dtype=torch.float32)
    zq = zp[:, :G, :] + sig.view(1, G, 1) * torch.randn((K, G, V), generator=g, device=device)
    zp = zp.to(tdtype)
    zq = zq.to(tdtype)
    drafts = _gumbel_argmax(zq, cfg.temp, g)
    return zp, zq, drafts


def generate(cfg: Config, device="cpu", B: int | None = None, data_seed: int | None = None,
             V: int | None = None, K: int | None = None, gamma: int | None = None,
             dtype: str | None = None):
    """Logits and drafts for a workload: dict(p [B,K,G+1,V], q [B,K,G,V], drafts [B,K,G]).

    Overrides (B, V, K, gamma, dtype) give smaller or ragged variants of a workload
    for parity tests.
    """
    B = cfg.B if B is None else B
    V = cfg.V if V is None else V
    K = cfg.K if K is None else K
    G = cfg.gamma if gamma is None else gamma
    dt = cfg.dtype if dtype is None else dtype
    ds = cfg.data_seed if data_seed is None else data_seed
    if dt not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16', got %r" % (dt,))
    tdtype = torch.float32 if dt == "f32" else torch.bfloat16
    p = torch.empty((B, K, G + 1, V), dtype=tdtype, device=device)
    q = torch.empty((B, K, G, V), dtype=tdtype, device=device)
    d = torch.empty((B, K, G), dtype=torch.int32, device=device)
    for b in range(B):
        zp, zq, dr = _one_prefix(cfg, b, ds, device, K, G, V, tdtype)
        p[b].copy_(zp)
        q[b].copy_(zq)
        d[b].copy_(dr)
    return {"p": p, "q": q, "drafts": d, "temp": cfg.temp, "dtype": dt}


def generate_pooled(cfg: Config, device="cpu", B: int | None = None,
                    data_seed: int | None = None, V: int | None = None, K: int | None = None,
                    gamma: int | None = None, dtype: str | None = None, tau: float | None = None):
    """Inputs with shared rows: dict(p_pool [NP,V], p_index [B,K,G+1], q_pool [B*G,V],
    q_index [B,K,G], drafts [B,K,G]).

    Recipe (per prefix b, own generator): position-j base logits 2 N(0,1) with
    a boosted mode token; one set of drafter rows z_q_j = base_j + sigma_j N(0,1)
    shared by the K drafts (one denoising pass exposes the marginals, and the K
    drafts are sampled from them); K drafts sampled independently from those
    rows; one verifier row per distinct draft prefix x_<j (a node of the draft
    tree, so row 0 is shared by all drafts), z_p = base_j + tau N(0,1).
    """
    B = cfg.B if B is None else B
    V = cfg.V if V is None else V
    K = cfg.K if K is None else K
    G = cfg.gamma if gamma is None else gamma
    dt = cfg.dtype if dtype is None else dtype
    ds = cfg.data_seed if data_seed is None else data_seed
    tau = cfg.tau if tau is None else tau
    if dt not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16', got %r" % (dt,))
    tdtype = torch.float32 if dt == "f32" else torch.bfloat16
    p_rows, q_rows = [], []
    p_index = torch.empty((B, K, G + 1), dtype=torch.int32)
    q_index = torch.empty((B, K, G), dtype=torch.int32)
    drafts = torch.empty((B, K, G), dtype=torch.int32, device=device)
    n_p = 0
    for b in range(B):
        g = _gen(device, ds * 1_000_003 + b)
        base = torch.randn((G + 1, V), generator=g, device=device, dtype=torch.float32) * 2.0
        mode = torch.randint(0, V, (G + 1, 1), generator=g, device=device)
        hit = torch.rand((G + 1, 1), generator=g, device=device) < cfg.boost_prob
        base.scatter_add_(-1, mode, hit.float() * cfg.boost)
        sig = cfg.sigma0 + cfg.sigma_step * torch.arange(G, device=device, dtype=torch.float32)
        zq = (base[:G] + sig.view(G, 1) * torch.randn((G, V), generator=g, device=device))
        zq = zq.to(tdtype)
        dr = _gumbel_argmax(zq.unsqueeze(0).expand(K, G, V), cfg.temp, g)
        drafts[b].copy_(dr)
        q_rows.append(zq)
        q_index[b] = (b * G + torch.arange(G, dtype=torch.int32)).view(1, G).expand(K, G)
        # one verifier row per node of the draft tree, in (position, first draft) order
        dh = dr.cpu().tolist()
        nodes, node_pos = {}, []
        for j in range(G + 1):
            for k in range(K):
                key = (j, tuple(dh[k][:j]))
                if key not in nodes:
                    nodes[key] = len(node_pos)
                    node_pos.append(j)
                p_index[b, k, j] = n_p + nodes[key]
        pos = torch.tensor(node_pos, device=device)
        zp = base[pos] + tau * torch.randn((len(node_pos), V), generator=g, device=device)
        p_rows.append(zp.to(tdtype))
        n_p += len(node_pos)
    return {"p_pool": torch.cat(p_rows, 0), "p_index": p_index.to(device),
            "q_pool": torch.cat(q_rows, 0), "q_index": q_index.to(device), "drafts": drafts,
            "temp": cfg.temp, "dtype": dt}


def tiny_trial_drafts(q_logits: torch.Tensor, n: int, temp: float, seed: int) -> torch.Tensor:
    """n independent draft sets for one logit instance: [n, K, gamma] int32.

    q_logits is [1, K, gamma, V]; every trial samples fresh tokens from it.
    """
    g = _gen(q_logits.device, seed)
    z = q_logits[0].float().unsqueeze(0).expand(n, *q_logits.shape[1:])
    return _gumbel_argmax(z, temp, g)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Host copy for the oracle: float32 stays float32, bf16 becomes its uint16 bit pattern."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    raise TypeError(t.dtype)
