"""Seeded random tensors (torch; any device).

Every tensor has its own stream, keyed by (seed, tensor id, sub id), so a
slice (one expert's weights) can be regenerated alone.  Values are standard
normal float32 draws from torch's generator for the chosen device, times the
tensor's standard deviation, then rounded to the storage dtype (bf16 rounding
is round-to-nearest-even).  The same device must be used to reproduce a
tensor: CPU and GPU generators give different (equally valid) streams.

Tensor ids: 1 router logits [T, E]; 2 activations x [T, H]; 3 expert
gate|up weights [E, 2I, H] (sub id = expert); 4 expert down weights [E, H, I]
(sub id = expert); 5 / 6 shared expert gate|up / down; 7 expert bias [E];
8 rank permutation for the skewed-load offsets; 9 output gradient dY;
10 router projection weight [E, H].
"""

import numpy as np
import torch

TID_LOGITS, TID_X, TID_W13, TID_W2, TID_SW13, TID_SW2, TID_BIAS, TID_RANK, TID_DY, TID_WR = range(1, 11)

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def tensor_seed(seed, tid, sub=0):
    """64-bit generator seed for (seed, tensor id, sub id)."""
    st = np.random.SeedSequence([int(seed), int(tid), int(sub)]).generate_state(2, dtype=np.uint32)
    return (int(st[0]) << 31) ^ int(st[1])


def randn(shape, std, dtype, device, seed, tid, sub=0, out=None):
    """N(0, std^2) tensor of `shape`, drawn in float32 then rounded to dtype."""
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(seed, tid, sub))
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    if out is not None:
        out.copy_(v)
        return out
    return v.to(_DT[dtype]) if isinstance(dtype, str) else v.to(dtype)


def zipf_offsets(E, s, beta, seed, device="cpu"):
    """Per-expert router-logit offsets o_e = -s * beta * ln(rank_e), centred,
    with ranks 1..E assigned by a seeded permutation.  Larger offsets make an
    expert more popular; the spread sets how skewed the per-expert load is."""
    g = torch.Generator(device="cpu")
    g.manual_seed(tensor_seed(seed, TID_RANK))
    rank = torch.randperm(E, generator=g).to(torch.float64) + 1.0
    o = -s * beta * torch.log(rank)
    o = o - o.mean()
    return o.to(torch.float32).to(device)


def expert_weights(cfg, which, device, seed=0, experts=None, dtype=None):
    """Weights of the listed experts (default all): which = 'w13' ([n, 2I, H])
    or 'w2' ([n, H, I]) or 'sw13' / 'sw2' for the shared expert (n = 1)."""
    H, I = cfg["H"], cfg["I"]
    dt = _DT[dtype or cfg["w_dtype"]]
    if which in ("sw13", "sw2"):
        Is = cfg["shared_I"]
        shape = (2 * Is, H) if which == "sw13" else (H, Is)
        tid = TID_SW13 if which == "sw13" else TID_SW2
        return randn((1,) + shape, cfg["w_std"], dt, device, seed, tid, 0)
    shape = (2 * I, H) if which == "w13" else (H, I)
    tid = TID_W13 if which == "w13" else TID_W2
    ids = range(cfg["E"]) if experts is None else experts
    ids = list(ids)
    out = torch.empty((len(ids),) + shape, dtype=dt, device=device)
    for j, e in enumerate(ids):
        out[j] = randn(shape, cfg["w_std"], torch.float32, device, seed, tid, e).to(dt)
    return out


def layer_inputs(cfg, device, seed=0, weights=True):
    """Activations, router logits, bias and (optionally) all weights."""
    T, H, E = cfg["T"], cfg["H"], cfg["E"]
    d = {}
    d["x"] = randn((T, H), 1.0, cfg["x_dtype"], device, seed, TID_X)
    logits = randn((T, E), 1.0, torch.float32, device, seed, TID_LOGITS)
    if cfg.get("zipf_beta"):
        logits = logits + zipf_offsets(E, 1.2, cfg["zipf_beta"], seed, device)[None, :]
    d["logits"] = logits.contiguous()
    d["bias"] = (randn((E,), cfg["bias_std"], torch.float32, device, seed, TID_BIAS)
                 if cfg.get("bias_std") else None)
    if weights:
        d["w13"] = expert_weights(cfg, "w13", device, seed)
        d["w2"] = expert_weights(cfg, "w2", device, seed)
        if cfg.get("shared_I"):
            d["sw13"] = expert_weights(cfg, "sw13", device, seed)
            d["sw2"] = expert_weights(cfg, "sw2", device, seed)
    return d


def output_grad(M, N, device, seed=0):
    """dY [M, N] bf16 N(0, 1) for the dgrad workload (rows in expert order)."""
    return randn((M, N), 1.0, "bf16", device, seed, TID_DY)


__all__ = ["tensor_seed", "randn", "zipf_offsets", "expert_weights", "layer_inputs",
           "output_grad"]


def router_weight(cfg, device, seed=0):
    """Router projection weight [E, H] float32, N(0, 1/H), so that the logits
    of N(0, 1) activations are about N(0, 1) like the generated logits."""
    return randn((cfg["E"], cfg["H"]), float(cfg["H"]) ** -0.5, torch.float32, device, seed, TID_WR)
