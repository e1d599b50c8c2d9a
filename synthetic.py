"""Seeded synthetic inputs shaped like the workloads the Bebop pages discuss.

This module is shared by the tests, the bench and the smoke check.  It holds none
of the method's arithmetic (no softmax, overlap, acceptance rule or sampling
rule): it only draws random logits with torch generators and draws draft tokens
from the stored draft logits by the Gumbel-max trick, argmax_v(z_v + G_v), which
samples softmax(z) without normalising it.

Workloads (gamma draft positions, vocabulary V):
  tiny          1 sequence, gamma = 3 (+1 bonus row), V = 1024, float32.
                target ~ N(0, 2^2); draft = target + N(0, 0.5^2).  The TV loss
                uses T = 1 with head k compared against target row k.
  rollout       64 sequences, gamma = 3 (+1 bonus row), V = 151936, bfloat16.
                target ~ N(0, 1) / 0.7; draft = target + N(0, 0.3^2).
  entropy_sweep 15 cells, tau in {0.25, 0.5, 1, 2, 4} x sigma in {0.1, 0.5, 1.0};
                128 sequences, gamma = 3 (+1 bonus row), V = 151936, bfloat16.
                target ~ N(0, 1) / tau; draft = target + N(0, sigma^2).
  tv_loss       T = 8192 positions, gamma = 3 heads, V = 151936, bfloat16.
                target ~ N(0, 1) / 0.8 shared by the heads; head k (1..3) =
                target + N(0, (0.2 k)^2).
  long_tail     512 sequences, gamma = 4 (+1 bonus row), V = 262144, bfloat16.
                target_v = -1.1 ln(pi_v) + N(0, 0.5^2) with pi a random
                permutation of the ranks 1..V per row (Zipf-like tail);
                draft = target + N(0, 0.4^2).
Draft noise is added to the unrounded target; both are then rounded once to the
storage dtype (round to nearest even for bfloat16).
"""
import torch

VERIFY_WORKLOADS = {
    "tiny": dict(B=1, G=3, V=1024, dtype=torch.float32, kind="normal", scale=2.0, sigma=0.5, seed=1),
    "rollout": dict(B=64, G=3, V=151936, dtype=torch.bfloat16, kind="normal", scale=1 / 0.7, sigma=0.3, seed=2),
    "long_tail": dict(B=512, G=4, V=262144, dtype=torch.bfloat16, kind="zipf", scale=0.5, sigma=0.4, seed=5),
}
SWEEP_TAUS = (0.25, 0.5, 1.0, 2.0, 4.0)
SWEEP_SIGMAS = (0.1, 0.5, 1.0)
TV_WORKLOADS = {
    "tiny": dict(T=1, G=3, V=1024, dtype=torch.float32, scale=2.0, sigma=0.5, shared=False, seed=1),
    "tv_loss": dict(T=8192, G=3, V=151936, dtype=torch.bfloat16, scale=1 / 0.8, sigma=0.2, shared=True, seed=4),
}


def sweep_cell(i_tau, i_sigma):
    """The entropy-sweep cell (tau index, sigma index) as a verify workload."""
    return dict(B=128, G=3, V=151936, dtype=torch.bfloat16, kind="normal", scale=1 / SWEEP_TAUS[i_tau],
                sigma=SWEEP_SIGMAS[i_sigma], seed=300 + 10 * i_tau + i_sigma)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _zipf_rows(n, V, noise, g, device, chunk=64):
    out = torch.empty((n, V), dtype=torch.float32, device=device)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        keys = torch.rand((e - s, V), generator=g, device=device)
        ranks = torch.argsort(keys, dim=1).to(torch.float32) + 1.0
        out[s:e] = -1.1 * torch.log(ranks) + noise * torch.randn((e - s, V), generator=g, device=device)
    return out


def gumbel_tokens(draft, g):
    """One draw per row from softmax(draft) (Gumbel-max), computed in float32 on the
    stored (rounded) logits.  draft: [..., V] -> int32 [...]."""
    u = torch.rand(draft.shape, generator=g, device=draft.device, dtype=torch.float32)
    gumbel = -torch.log(-torch.log(u.clamp_min(1e-38)))
    return torch.argmax(draft.to(torch.float32) + gumbel, dim=-1).to(torch.int32)


def verify_inputs(w, device="cpu", seed=None, B=None, V=None, chunk=16):
    """(target [B, G+1, V], draft [B, G, V], draft_tokens int32 [B, G]) for a verify
    workload dict (see VERIFY_WORKLOADS / sweep_cell).  B, V and seed override."""
    B = w["B"] if B is None else B
    V = w["V"] if V is None else V
    G = w["G"]
    g = _gen(device, w["seed"] if seed is None else seed)
    target = torch.empty((B, G + 1, V), dtype=w["dtype"], device=device)
    draft = torch.empty((B, G, V), dtype=w["dtype"], device=device)
    tokens = torch.empty((B, G), dtype=torch.int32, device=device)
    for s in range(0, B, chunk):
        e = min(B, s + chunk)
        n = e - s
        if w["kind"] == "zipf":
            t = _zipf_rows(n * (G + 1), V, w["scale"], g, device).view(n, G + 1, V)
        else:
            t = w["scale"] * torch.randn((n, G + 1, V), generator=g, device=device)
        d = t[:, :G] + w["sigma"] * torch.randn((n, G, V), generator=g, device=device)
        target[s:e] = t.to(w["dtype"])
        draft[s:e] = d.to(w["dtype"])
        tokens[s:e] = gumbel_tokens(draft[s:e], g)
    return target, draft, tokens


def tv_inputs(w, device="cpu", seed=None, T=None, V=None, chunk=256):
    """(target, draft) for a TV-loss workload: target [T, V] when shared by the
    heads, else [T, G, V]; draft [T, G, V]."""
    T = w["T"] if T is None else T
    V = w["V"] if V is None else V
    G = w["G"]
    g = _gen(device, w["seed"] if seed is None else seed)
    shared = w["shared"]
    target = torch.empty((T, V) if shared else (T, G, V), dtype=w["dtype"], device=device)
    draft = torch.empty((T, G, V), dtype=w["dtype"], device=device)
    heads = torch.arange(1, G + 1, device=device, dtype=torch.float32).view(1, G, 1)
    for s in range(0, T, chunk):
        e = min(T, s + chunk)
        n = e - s
        if shared:
            t = w["scale"] * torch.randn((n, V), generator=g, device=device)
            base = t[:, None, :]
            d = base + (w["sigma"] * heads) * torch.randn((n, G, V), generator=g, device=device)
        else:
            t = w["scale"] * torch.randn((n, G, V), generator=g, device=device)
            d = t + w["sigma"] * torch.randn((n, G, V), generator=g, device=device)
        target[s:e] = t.to(w["dtype"])
        draft[s:e] = d.to(w["dtype"])
    return target, draft


def topk_inputs(w, K, device="cpu", seed=None, T=None, V=None):
    """(target_idx int32, target_val float32, draft) for the top-K TV path: a TV
    workload's target rows reduced to their K largest logits (indices and the
    stored values, widened to float32), [T, K] when shared by the heads, else
    [T, G, K]; the draft as in tv_inputs."""
    target, draft = tv_inputs(w, device, seed=seed, T=T, V=V)
    val, idx = torch.topk(target.to(torch.float32), K, dim=-1)
    return idx.to(torch.int32).contiguous(), val.contiguous(), draft
