"""Seeded synthetic inputs for the verify-and-sample step and the MTP shift.

This module only draws random inputs.  It holds none of the verification
arithmetic (no softmax, no acceptance test, no inverse CDF, no shift).  The GPU
parity tests, the CPU oracle tests and the benchmark all take their inputs from
here, so both sides of every comparison see the same tensors.

Workload shapes follow the configurations the benchmark and tests use:

  1  tiny sampling:        B=1,    n=4, V=32000,  fp32, T=1.0, L=4
  2  Llama-vocab sampling: B=64,   n=4, V=128256, bf16, T=0.7, L ~ U{1..4}
  3  greedy + MTP shift:   B=256,  n=4, V=128256, bf16, greedy, L=4, H=8192
  4  single-token MTP:     B=512,  n=1, V=129280, bf16, T=0.6, L=1, H=7168
  5  long ragged drafts:   B=1024, n=8, V=152064, bf16, T in {0,0.7,1}, L ~ U{0..8}
  6  recipe 2 at B=256:    B=256,  n=4, V=128256, bf16, T=0.7, L ~ U{1..4}

and make_lmhead() draws hidden states and a logit projection (instead of
logits) for the fused projection + greedy verify, B=256, n=4, V=128256, H=8192
by default.

Draft tokens for sampling sequences are drawn from the draft distribution
softmax(z_d / T) with the Gumbel-max construction (argmax of z_d / T plus
Gumbel noise): this is the draft model's own sampling, which precedes the step.
Greedy sequences (T = 0) draft the argmax of the draft logits.  For the greedy
configuration the target's top token is planted at a random index of every row,
so the draft can "match the target argmax" without this module computing it.

Every tensor is produced by a torch.Generator seeded with the given seed on the
given device; no step depends on the code under test.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int
    n: int
    V: int
    dtype: torch.dtype
    H: int = 0            # hidden size of the MTP carry (0: no hidden buffer)
    mode: str = "sample"  # "sample" or "greedy"


CONFIGS = {
    1: Config(1, "tiny_sampling_fp32", 1, 4, 32000, torch.float32),
    2: Config(2, "llama_vocab_sampling", 64, 4, 128256, torch.bfloat16),
    3: Config(3, "greedy_verify_mtp_shift", 256, 4, 128256, torch.bfloat16, H=8192, mode="greedy"),
    4: Config(4, "single_token_mtp", 512, 1, 129280, torch.bfloat16, H=7168),
    5: Config(5, "long_ragged_drafts", 1024, 8, 152064, torch.bfloat16),
    # the llama-vocab sampling recipe at B=256, n=4, V=128256 (the greedy workload's shape)
    6: Config(6, "llama_vocab_sampling_b256", 256, 4, 128256, torch.bfloat16),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _gumbel_draft(zd: torch.Tensor, T: torch.Tensor, g: torch.Generator) -> torch.Tensor:
    """Draft tokens drawn from softmax(zd / T) by Gumbel-max; zd [b, n, V]."""
    u = torch.rand(zd.shape, generator=g, device=zd.device, dtype=torch.float32)
    u.clamp_(min=1e-12, max=1.0 - 1e-7)
    gumbel = -torch.log(-torch.log(u))
    scaled = zd.float() / T.view(-1, 1, 1)
    return torch.argmax(scaled + gumbel, dim=-1).to(torch.int32)


def make(cid: int, seed: int, device="cpu", B: int | None = None, V: int | None = None,
         H: int | None = None, n: int | None = None, block: int = 64) -> dict:
    """Inputs of configuration ``cid`` (shape overrides allowed for small cases).

    Returns a dict of tensors on ``device``:
      target [B, n+1, V], draft [B, n, V] (None in greedy mode), draft_tokens [B, n],
      draft_lens [B], temperature [B], uniforms [B, n+1], tokens [B, n+1] (MTP
      token buffer: slot 0 the last committed token, slots 1..n the drafts),
      hidden [B, n+1, H] (when H > 0).
    """
    cfg = CONFIGS[cid]
    rc = 2 if cid == 6 else cid  # the recipe
    B = cfg.B if B is None else B
    V = cfg.V if V is None else V
    n = cfg.n if n is None else n
    H = cfg.H if H is None else H
    dev = torch.device(device)
    g = _gen(seed, dev)
    dt = cfg.dtype

    target = torch.empty((B, n + 1, V), dtype=dt, device=dev)
    draft = None if cfg.mode == "greedy" else torch.empty((B, n, V), dtype=dt, device=dev)
    draft_tokens = torch.empty((B, n), dtype=torch.int32, device=dev)

    # per-sequence scalars first (small), drawn in a fixed order
    if rc == 1:
        lens = torch.full((B,), n, dtype=torch.int32, device=dev)
        temp = torch.full((B,), 1.0, dtype=torch.float32, device=dev)
        sigma = torch.full((B,), 0.5, device=dev)
        scale = 2.0
    elif rc == 2:
        lens = torch.randint(1, n + 1, (B,), generator=g, device=dev, dtype=torch.int32) if n > 0 \
            else torch.zeros(B, dtype=torch.int32, device=dev)
        temp = torch.full((B,), 0.7, dtype=torch.float32, device=dev)
        sigma = torch.full((B,), 1.0, device=dev)
        scale = 3.0
    elif rc == 3:
        lens = torch.full((B,), n, dtype=torch.int32, device=dev)
        temp = torch.zeros((B,), dtype=torch.float32, device=dev)
        sigma = None
        scale = 3.0
    elif rc == 4:
        lens = torch.full((B,), n, dtype=torch.int32, device=dev)
        temp = torch.full((B,), 0.6, dtype=torch.float32, device=dev)
        sigma = torch.full((B,), 0.7, device=dev)
        scale = 3.0
    elif rc == 5:
        lens = torch.randint(0, n + 1, (B,), generator=g, device=dev, dtype=torch.int32)
        choices = torch.tensor([0.0, 0.7, 1.0], device=dev)
        temp = choices[torch.randint(0, 3, (B,), generator=g, device=dev)].to(torch.float32)
        sigma = 0.3 + 1.7 * torch.rand((B,), generator=g, device=dev)
        scale = 3.0
    else:
        raise ValueError(cid)

    for b0 in range(0, B, block):
        b1 = min(B, b0 + block)
        nb = b1 - b0
        zt = scale * torch.randn((nb, n + 1, V), generator=g, device=dev, dtype=torch.float32)
        if rc == 2 and V > 20:
            # top-20 boost: the 20 largest logits of each target row gain +6
            top = torch.topk(zt, 20, dim=-1).indices
            zt.scatter_add_(-1, top, torch.full(top.shape, 6.0, device=dev))
        if rc == 3:
            # plant the row's top token (in 1/8 of rows also a tied twin)
            rows = nb * (n + 1)
            ztf = zt.view(rows, V)
            a_top = torch.randint(0, V, (rows,), generator=g, device=dev)
            a_tie = (a_top + 1 + torch.randint(0, max(V - 1, 1), (rows,), generator=g, device=dev)) % V
            tie = torch.rand((rows,), generator=g, device=dev) < 0.125
            level = 20.0 + 4.0 * torch.rand((rows,), generator=g, device=dev)
            r = torch.arange(rows, device=dev)
            ztf[r, a_top] = level
            ztf[r[tie], a_tie[tie]] = level[tie]
            target[b0:b1] = zt.to(dt)
            # drafts: the planted top (or its twin, evenly) with probability 0.7,
            # otherwise a uniform index other than the planted top
            a_top = a_top.view(nb, n + 1)[:, :n]
            a_tie = a_tie.view(nb, n + 1)[:, :n]
            tie = tie.view(nb, n + 1)[:, :n]
            hit = torch.rand((nb, n), generator=g, device=dev) < 0.7
            pick_twin = tie & (torch.rand((nb, n), generator=g, device=dev) < 0.5)
            match = torch.where(pick_twin, a_tie, a_top)
            other = torch.randint(0, max(V - 1, 1), (nb, n), generator=g, device=dev)
            other = torch.where(other >= a_top, other + 1, other) % V
            draft_tokens[b0:b1] = torch.where(hit, match, other).to(torch.int32)
            continue
        target[b0:b1] = zt.to(dt)
        zt_r = target[b0:b1, :n].float()                       # the values both sides read
        noise = torch.randn((nb, n, V), generator=g, device=dev, dtype=torch.float32)
        zd = (zt_r + sigma[b0:b1].view(-1, 1, 1) * noise).to(dt)
        draft[b0:b1] = zd
        tb = temp[b0:b1]
        greedy_rows = tb == 0
        tsafe = torch.where(greedy_rows, torch.ones_like(tb), tb)
        x = _gumbel_draft(zd, tsafe, g) if n > 0 else torch.empty((nb, 0), dtype=torch.int32, device=dev)
        if greedy_rows.any() and n > 0:
            xg = torch.argmax(zd.float(), dim=-1).to(torch.int32)
            x = torch.where(greedy_rows.view(-1, 1), xg, x)
        draft_tokens[b0:b1] = x
        del zt, zt_r, noise, zd

    uniforms = torch.rand((B, n + 1), generator=g, device=dev, dtype=torch.float32)
    first = torch.randint(0, V, (B, 1), generator=g, device=dev, dtype=torch.int32)
    tokens = torch.cat([first, draft_tokens], dim=1).contiguous()
    out = dict(cfg=cfg, B=B, n=n, V=V, target=target, draft=draft, draft_tokens=draft_tokens,
               draft_lens=lens, temperature=temp, uniforms=uniforms, tokens=tokens)
    if H:
        out["hidden"] = torch.randn((B, n + 1, H), generator=g, device=dev,
                                    dtype=torch.float32).to(torch.bfloat16)
    out["H"] = H
    return out


def tree_parents(n: int, widths=(3, 2, 1)) -> list:
    """Parents of nodes 1..n of a top-k style draft tree, built level by level:
    a node at depth d gets up to widths[d] children (1 beyond the listed depths),
    so the tree is bushy near the root and thins to chains.  Entry j is the
    parent of node j + 1."""
    par, depth, q = [], [0], [0]
    while len(par) < n and q:
        nxt = []
        for node in q:
            w = widths[depth[node]] if depth[node] < len(widths) else 1
            for _ in range(w):
                if len(par) == n:
                    break
                par.append(node)
                depth.append(depth[node] + 1)
                nxt.append(len(par))
        q = nxt
    return par


def make_tree(seed: int, device="cpu", B: int = 64, n: int = 25, V: int = 128256, shape: str = "topk",
              dtype=torch.bfloat16, ragged: bool = False) -> dict:
    """Inputs of greedy tree verification: target logits [B, n+1, V] (row r = the
    target's logits after node r) drawn like the greedy logits recipe (N(0, 3^2)
    with every row's top token planted at a random index, in 1/8 of rows also a
    tied twin), draft_parents [B, n] (shape "topk": tree_parents(n) for every
    sequence; "random": node j + 1 below a uniform node in [0, j]), draft_tokens
    [B, n]: among each node's children one, chosen at random, carries the node's
    planted top (or its twin) with probability 0.8; the others carry other
    tokens.  draft_lens [B]: n, or uniform in 0..n when ragged."""
    import numpy as np

    dev = torch.device(device)
    g = _gen(seed, dev)
    rows = B * (n + 1)
    zt = 3.0 * torch.randn((rows, V), generator=g, device=dev, dtype=torch.float32)
    a_top = torch.randint(0, V, (rows,), generator=g, device=dev)
    a_tie = (a_top + 1 + torch.randint(0, max(V - 1, 1), (rows,), generator=g, device=dev)) % V
    tie = torch.rand((rows,), generator=g, device=dev) < 0.125
    level = 20.0 + 4.0 * torch.rand((rows,), generator=g, device=dev)
    r = torch.arange(rows, device=dev)
    zt[r, a_top] = level
    zt[r[tie], a_tie[tie]] = level[tie]
    target = zt.view(B, n + 1, V).to(dtype)
    top = a_top.view(B, n + 1).cpu().numpy()
    twin = a_tie.view(B, n + 1).cpu().numpy()
    has_twin = tie.view(B, n + 1).cpu().numpy()
    rng = np.random.default_rng(seed)
    if shape == "topk":
        par = np.tile(np.array(tree_parents(n), dtype=np.int32), (B, 1)) if n > 0 else np.zeros((B, 0), np.int32)
    else:
        par = np.array([[rng.integers(0, j + 1) for j in range(n)] for _ in range(B)], dtype=np.int32).reshape(B, n)
    tok = np.empty((B, n), dtype=np.int64)
    for b in range(B):
        for p in np.unique(par[b]):
            kids = np.nonzero(par[b] == p)[0]
            hit = kids[rng.integers(0, len(kids))] if rng.random() < 0.8 else -1
            for j in kids:
                if j == hit:
                    tok[b, j] = twin[b, p] if has_twin[b, p] and rng.random() < 0.5 else top[b, p]
                else:
                    o = int(rng.integers(0, max(V - 1, 1)))
                    tok[b, j] = (o + 1) % V if o >= top[b, p] else o
    lens = rng.integers(0, n + 1, B) if ragged else np.full(B, n)
    return dict(target=target, draft_parents=torch.as_tensor(par, dtype=torch.int32, device=dev),
                draft_tokens=torch.as_tensor(tok, dtype=torch.int32, device=dev),
                draft_lens=torch.as_tensor(lens, dtype=torch.int32, device=dev), B=B, n=n, V=V)


def make_tree_sample(seed: int, device="cpu", B: int = 64, n: int = 25, V: int = 128256, shape: str = "topk",
                     dtype=torch.bfloat16, ragged: bool = False, temps=(0.7,), sigma: float = 1.0,
                     block: int = 16) -> dict:
    """Inputs of sampling tree verification.  Target row r [B, n+1, V] (the
    target after node r) follows the llama-vocab sampling recipe: N(0, 3^2) with
    the row's 20 largest logits raised by 6.  Draft row r [B, n, V] is the
    target row r as stored plus N(0, sigma^2).  draft_parents as in make_tree
    ("topk": tree_parents(n); "random": node j + 1 below a uniform node in
    [0, j]); node j + 1's token is drawn from softmax(draft row parent / T) by
    Gumbel-max, independently for every child (the draft's own sampling), or
    is the argmax of that row when T = 0.  temperature: uniform over `temps`;
    draft_lens: n, or uniform in 0..n when ragged; uniforms [B, n+1]."""
    import numpy as np

    dev = torch.device(device)
    g = _gen(seed, dev)
    rng = np.random.default_rng(seed)
    if shape == "topk":
        par = np.tile(np.array(tree_parents(n), dtype=np.int32), (B, 1)) if n > 0 else np.zeros((B, 0), np.int32)
    else:
        par = np.array([[rng.integers(0, j + 1) for j in range(n)] for _ in range(B)], dtype=np.int32).reshape(B, n)
    tv = torch.tensor([float(t) for t in temps], device=dev)
    temp = tv[torch.randint(0, len(temps), (B,), generator=g, device=dev)].to(torch.float32)
    lens = torch.randint(0, n + 1, (B,), generator=g, device=dev, dtype=torch.int32) if ragged \
        else torch.full((B,), n, dtype=torch.int32, device=dev)
    target = torch.empty((B, n + 1, V), dtype=dtype, device=dev)
    draft = torch.empty((B, n, V), dtype=dtype, device=dev)
    tokens = torch.empty((B, n), dtype=torch.int32, device=dev)
    parents = torch.as_tensor(par, dtype=torch.int32, device=dev)
    for b0 in range(0, B, block):
        b1 = min(B, b0 + block)
        nb = b1 - b0
        zt = 3.0 * torch.randn((nb, n + 1, V), generator=g, device=dev, dtype=torch.float32)
        if V > 20:
            top = torch.topk(zt, 20, dim=-1).indices
            zt.scatter_add_(-1, top, torch.full(top.shape, 6.0, device=dev))
        target[b0:b1] = zt.to(dtype)
        del zt
        noise = torch.randn((nb, n, V), generator=g, device=dev, dtype=torch.float32)
        draft[b0:b1] = (target[b0:b1, :n].float() + sigma * noise).to(dtype)
        del noise
        if n == 0:
            continue
        tb = temp[b0:b1]
        greedy = tb == 0
        tsafe = torch.where(greedy, torch.ones_like(tb), tb)
        pr = parents[b0:b1].long()
        at_parent = draft[b0:b1].gather(1, pr.unsqueeze(-1).expand(nb, n, V))   # draft row of each node's parent
        x = _gumbel_draft(at_parent, tsafe, g)
        xg = torch.argmax(at_parent.float(), dim=-1).to(torch.int32)
        tokens[b0:b1] = torch.where(greedy.view(-1, 1), xg, x)
        del at_parent
    uniforms = torch.rand((B, n + 1), generator=g, device=dev, dtype=torch.float32)
    return dict(target=target, draft=draft, draft_tokens=tokens, draft_parents=parents, draft_lens=lens,
                temperature=temp, uniforms=uniforms, B=B, n=n, V=V, parents_host=par)


def make_lmhead(seed: int, device="cpu", B: int = 256, n: int = 4, V: int = 128256, H: int = 8192,
                exact: bool = True, ragged: bool = False) -> dict:
    """Inputs of the fused logit projection + greedy verify: the target's final
    hidden states and its logit projection instead of materialised logits.

    Returns hidden [B, n+1, H] bf16, weight [V, H] bf16 (one row per vocabulary
    entry), draft_tokens [B, n], draft_lens [B], tokens [B, n+1] (MTP buffer).

    exact=True: every hidden value is an integer in [-R, R] times 2^-4 and every
    weight an integer in [-R, R] times 2^-e, with R = min(44, sqrt(2^24 / H)) and
    e chosen so that the logits have a standard deviation near 3.  Every partial
    sum of a logit is then an integer multiple of 2^-(4+e) below 2^24 such
    units in magnitude, exactly representable in binary32, so the logits (and
    their argmax) do not depend on the order of summation.
    exact=False: weight ~ N(0, 9/H) and hidden ~ N(0, 1) (logits ~ N(0, 9)).

    As in the greedy logits recipe, each row's top token is planted: hidden row
    m leans towards weight row a_m (its logit sits about 6.5 standard deviations
    above the mean), and in 1/8 of rows a twin index receives a copy of weight
    row a_m, so the two logits tie exactly in every row.  Drafts are the planted
    top (or its twin) with probability 0.7, otherwise another index.
    """
    dev = torch.device(device)
    g = _gen(seed, dev)
    M = B * (n + 1)
    if exact:
        R = int(min(44, math.isqrt((1 << 24) // H)))
        Wi = torch.randint(-R, R + 1, (V, H), generator=g, device=dev, dtype=torch.int16)
    else:
        Wf = (3.0 / math.sqrt(H)) * torch.randn((V, H), generator=g, device=dev, dtype=torch.float32)
    a_top = torch.randint(0, V, (M,), generator=g, device=dev)
    a_tie = (a_top + 1 + torch.randint(0, max(V - 1, 1), (M,), generator=g, device=dev)) % V
    tie = (torch.rand((M,), generator=g, device=dev) < 0.125) & (V > 1)
    W = Wi if exact else Wf
    for m in torch.nonzero(tie).flatten().tolist():  # in row order: later copies win
        W[a_tie[m]] = W[a_top[m]]
    if exact:
        noise = torch.randint(-R + 3, R - 2, (M, H), generator=g, device=dev, dtype=torch.int16)
        # the lean adds about lam * H * var(w) units to the planted logit: 6.5 standard deviations
        lam = 6.5 * math.sqrt(((2 * R - 5) ** 2 - 1) / 12.0) / (math.sqrt(H) * math.sqrt((((2 * R + 1) ** 2) - 1) / 12.0))
        lean = torch.round(lam * Wi[a_top].float()).to(torch.int16)
        a = torch.clamp(noise + lean, -R, R)
        hidden = (a.float() * 2.0 ** -4).to(torch.bfloat16)
        var_w = (((2 * R + 1) ** 2) - 1) / 12.0
        var_h = (((2 * R - 5) ** 2) - 1) / 12.0
        e = round(math.log2(math.sqrt(H * var_h * var_w) / 16.0 / 3.0))
        weight = (Wi.float() * 2.0 ** -e).to(torch.bfloat16)
        del Wi, noise, lean, a
    else:
        mu = 6.5 / math.sqrt(H)
        hidden = (torch.randn((M, H), generator=g, device=dev) + mu * Wf[a_top] * (math.sqrt(H) / 3.0))
        hidden = hidden.to(torch.bfloat16)
        weight = Wf.to(torch.bfloat16)
        del Wf
    hidden = hidden.view(B, n + 1, H)
    if ragged:
        lens = torch.randint(0, n + 1, (B,), generator=g, device=dev, dtype=torch.int32)
    else:
        lens = torch.full((B,), n, dtype=torch.int32, device=dev)
    top = a_top.view(B, n + 1)[:, :n]
    twin = a_tie.view(B, n + 1)[:, :n]
    tie = tie.view(B, n + 1)[:, :n]
    hit = torch.rand((B, n), generator=g, device=dev) < 0.7
    pick_twin = tie & (torch.rand((B, n), generator=g, device=dev) < 0.5)
    match = torch.where(pick_twin, twin, top)
    other = torch.randint(0, max(V - 1, 1), (B, n), generator=g, device=dev)
    other = torch.where(other >= top, other + 1, other) % V
    draft_tokens = torch.where(hit, match, other).to(torch.int32)
    first = torch.randint(0, V, (B, 1), generator=g, device=dev, dtype=torch.int32)
    tokens = torch.cat([first, draft_tokens], dim=1).contiguous()
    return dict(B=B, n=n, V=V, H=H, hidden=hidden.contiguous(), weight=weight.contiguous(),
                draft_tokens=draft_tokens.contiguous(), draft_lens=lens, tokens=tokens)


def make_law_case(seed: int, trials: int, V: int = 8, n: int = 4, T: float = 1.0,
                  draft_sigma: float = 1.0, device="cpu") -> dict:
    """Many trials of one fixed set of rows (for distribution-law tests).

    Target rows [n+1, V] and draft rows [n, V] are drawn once from the seed and
    repeated for every trial; each trial gets fresh draft tokens drawn from the
    draft distribution and fresh uniforms.  fp32 logits.
    """
    dev = torch.device(device)
    g = _gen(seed, dev)
    zt = 1.5 * torch.randn((n + 1, V), generator=g, device=dev)
    zd = zt[:n] + draft_sigma * torch.randn((n, V), generator=g, device=dev)
    target = zt.expand(trials, n + 1, V).contiguous()
    draft = zd.expand(trials, n, V).contiguous()
    temp = torch.full((trials,), float(T), device=dev)
    x = _gumbel_draft(draft, temp, g)
    uniforms = torch.rand((trials, n + 1), generator=g, device=dev)
    lens = torch.full((trials,), n, dtype=torch.int32, device=dev)
    return dict(target=target, draft=draft, draft_tokens=x, draft_lens=lens, temperature=temp,
                uniforms=uniforms, rows_t=zt, rows_d=zd, T=T, B=trials, n=n, V=V)


def make_tree_law_case(seed: int, trials: int, V: int = 8, widths=(3, 2), T: float = 1.0, draft_sigma: float = 1.0,
                       device="cpu") -> dict:
    """Many trials of sampling tree verification on one two-level draft tree
    (widths[0] children of the root, widths[1] below each), fp32 logits.

    The target's and the draft's logits after a node depend only on the tokens
    on the way to it (tables drawn once from the seed: z0 for the root, z1[v]
    after token v, z2[v][w] after v then w; draft = target + N(0, sigma^2)), as
    they do for a real model.  Each trial draws the children of every node
    independently from the draft's distribution at that node (Gumbel-max on the
    draft logits / T) and its own uniforms.  Returns the step's inputs (target
    [trials, n+1, V], draft [trials, n, V], draft_tokens, draft_parents,
    draft_lens, temperature, uniforms) and the tables rows_t0, rows_t1, rows_t2.
    """
    dev = torch.device(device)
    g = _gen(seed, dev)
    k1, k2 = widths
    par = tree_parents(k1 + k1 * k2, widths=(k1, k2, 0))
    n = len(par)
    z0 = 1.5 * torch.randn((V,), generator=g, device=dev)
    d0 = z0 + draft_sigma * torch.randn((V,), generator=g, device=dev)
    z1 = 1.5 * torch.randn((V, V), generator=g, device=dev)
    d1 = z1 + draft_sigma * torch.randn((V, V), generator=g, device=dev)
    z2 = 1.5 * torch.randn((V, V, V), generator=g, device=dev)
    d2 = z2 + draft_sigma * torch.randn((V, V, V), generator=g, device=dev)
    temp = torch.full((trials,), float(T), device=dev)
    # children of the root, then k2 children below each of them
    x1 = _gumbel_draft(d0.expand(trials, k1, V), temp, g).long()                    # [trials, k1]
    x2 = _gumbel_draft(d1[x1].repeat_interleave(k2, dim=1), temp, g).long()
    x2 = x2.view(trials, k1, k2)
    tokens = torch.cat([x1, x2.reshape(trials, k1 * k2)], dim=1)                     # node order of tree_parents
    target = torch.empty((trials, n + 1, V), device=dev)
    draft = torch.empty((trials, n, V), device=dev)
    target[:, 0] = z0
    draft[:, 0] = d0
    target[:, 1:1 + k1] = z1[x1]
    draft[:, 1:1 + k1] = d1[x1]
    v = x1.repeat_interleave(k2, dim=1)                                               # parent token of each leaf
    w = x2.reshape(trials, k1 * k2)
    target[:, 1 + k1:] = z2[v, w]
    draft[:, 1 + k1:] = d2[v, w][:, :n - 1 - k1]                                     # leaves' rows (unused)
    uniforms = torch.rand((trials, n + 1), generator=g, device=dev)
    return dict(target=target, draft=draft, draft_tokens=tokens.to(torch.int32),
                draft_parents=torch.as_tensor(par, dtype=torch.int32, device=dev).expand(trials, n).contiguous(),
                draft_lens=torch.full((trials,), n, dtype=torch.int32, device=dev), temperature=temp,
                uniforms=uniforms, rows_t0=z0, rows_t1=z1, rows_t2=z2, B=trials, n=n, V=V, T=T, widths=widths)


def make_tree_law_case3(seed: int, trials: int, V: int = 4, draft_sigma: float = 1.0, T: float = 1.0,
                        device="cpu") -> dict:
    """make_tree_law_case on a three-level binary tree (2 candidates at every
    inner node, 14 candidates; nodes numbered level by level as tree_parents
    does).  Tables z0, z1[a], z2[a][b], z3[a][b][c] (the target after the token
    prefix; N(0, 1.5^2)) and the draft's (+ N(0, sigma^2)); every trial draws
    each inner node's 2 children independently from the draft at that node."""
    dev = torch.device(device)
    g = _gen(seed, dev)
    par = tree_parents(14, widths=(2, 2, 2, 0))
    n = len(par)
    zs, ds = [], []
    for k in range(4):
        z = 1.5 * torch.randn((V,) * (k + 1), generator=g, device=dev)
        zs.append(z)
        ds.append(z + draft_sigma * torch.randn((V,) * (k + 1), generator=g, device=dev))
    temp = torch.full((trials,), float(T), device=dev)

    def draw(rows):  # rows [trials, m, V]: one Gumbel-max draw from each
        return _gumbel_draft(rows, temp, g).long()

    x1 = draw(ds[0].expand(trials, 2, V))                                         # nodes 1, 2
    x2 = draw(ds[1][x1].repeat_interleave(2, dim=1))                              # nodes 3..6
    a2 = x1.repeat_interleave(2, dim=1)                                           # their parents' tokens
    x3 = draw(ds[2][a2, x2].repeat_interleave(2, dim=1))                          # nodes 7..14
    a3, b3 = a2.repeat_interleave(2, dim=1), x2.repeat_interleave(2, dim=1)
    tokens = torch.cat([x1, x2, x3], dim=1)
    target = torch.empty((trials, n + 1, V), device=dev)
    draft = torch.empty((trials, n, V), device=dev)
    target[:, 0], draft[:, 0] = zs[0], ds[0]
    target[:, 1:3], draft[:, 1:3] = zs[1][x1], ds[1][x1]
    target[:, 3:7], draft[:, 3:7] = zs[2][a2, x2], ds[2][a2, x2]
    target[:, 7:15] = zs[3][a3, b3, x3]
    draft[:, 7:14] = ds[3][a3, b3, x3][:, :7]                                    # leaves' rows (unused)
    uniforms = torch.rand((trials, n + 1), generator=g, device=dev)
    return dict(target=target, draft=draft, draft_tokens=tokens.to(torch.int32),
                draft_parents=torch.as_tensor(par, dtype=torch.int32, device=dev).expand(trials, n).contiguous(),
                draft_lens=torch.full((trials,), n, dtype=torch.int32, device=dev), temperature=temp,
                uniforms=uniforms, tables=zs, B=trials, n=n, V=V, T=T)


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bfloat16 tensor (for the oracle)."""
    import numpy as np
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_logits(t: torch.Tensor):
    """numpy array the oracle accepts: fp32 as float32, bf16 as uint16 bits."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().cpu().contiguous().numpy()


def expected_rows(cfg: Config) -> float:
    """Mean number of logit rows a step reads for the config's recipe."""
    n = cfg.n
    if cfg.cid == 1:
        return 2 * n + 1
    if cfg.cid in (2, 6):
        return sum((L + 1) + L for L in range(1, n + 1)) / n * cfg.B
    if cfg.cid == 3:
        return (n + 1) * cfg.B
    if cfg.cid == 4:
        return (2 * n + 1) * cfg.B
    if cfg.cid == 5:
        per = sum((L + 1) + (2.0 / 3.0) * L for L in range(0, n + 1)) / (n + 1)
        return per * cfg.B
    return math.nan
