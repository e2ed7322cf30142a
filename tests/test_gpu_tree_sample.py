"""GPU parity of sampling tree verification (spec_verify_tree_sample) against
the oracle (SpecInfer's multi-step speculative sampling on the draft tree).

Every sequence is compared in full: accepted length, emitted tokens, kept path
and the OR of the flags.  A sequence may differ only when the oracle's margin
of one of its decisions (|u - ratio| of a test, the draw's distance to a CDF
boundary over the residual's mass) is below 1e-5, the rounding band between a
float kernel and a double/extended-precision oracle; it is then counted as
exempt.  Cases: random and top-k trees over several tiles with a ragged tail,
bf16 and fp32, temperatures 0 / 0.7 / 1 mixed in one batch; round limits that
truncate walks (compared with the oracle under the same limit); the top-k tree
at full size (B = 64, 26 nodes, V = 128256); the chain tree against the linear
call; bad parents, tokens and lengths; the workspace left zero-filled.
"""
import numpy as np
import pytest
import torch

import draft_token_verification_08_amd as sv
from draft_token_verification_08_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-5


def _rounds(d):
    par = d["parents_host"] if "parents_host" in d else d["draft_parents"].cpu().numpy()
    return max([sv.sv_tree_rounds(list(p)) for p in par] + [0])


def _run(d, max_rounds, ws=None):
    fl = torch.zeros(1, dtype=torch.int32, device=DEV)
    acc, emi, path = sv.spec_verify_tree_sample(d["target"], d["draft"], d["draft_tokens"], d["draft_parents"],
                                                d["draft_lens"], d["temperature"], d["uniforms"], max_rounds,
                                                err_flags=fl, workspace=ws)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), emi.cpu().numpy(), path.cpu().numpy(), int(fl.item())


def _oracle(oracle, d, max_rounds=None):
    return oracle.verify_tree_sample(synth.host_logits(d["target"]), synth.host_logits(d["draft"]),
                                     d["draft_tokens"].cpu().numpy(), d["draft_parents"].cpu().numpy(),
                                     d["draft_lens"].cpu().numpy(), d["temperature"].cpu().numpy(),
                                     d["uniforms"].cpu().numpy(), max_rounds=max_rounds)


def _compare(oracle, d, max_rounds, oracle_rounds="same", ws=None, tag=""):
    acc, emi, path, fl = _run(d, max_rounds, ws)
    o = _oracle(oracle, d, max_rounds if oracle_rounds == "same" else oracle_rounds)
    B = acc.shape[0]
    temp = d["temperature"].cpu().numpy()
    am, dm = o["accept_margin"], o["draw_margin"]
    exempt = hard = 0
    first = None
    for b in range(B):
        same = (acc[b] == o["accepted_len"][b] and np.array_equal(emi[b], o["emitted"][b])
                and np.array_equal(path[b], o["path"][b]))
        if same:
            continue
        tie = temp[b] > 0 and ((am[b] < TOL).any() or dm[b] < TOL)
        if tie:
            exempt += 1
            continue
        hard += 1
        if first is None:
            first = (b, int(acc[b]), int(o["accepted_len"][b]), emi[b].tolist(), o["emitted"][b].tolist(),
                     path[b].tolist(), o["path"][b].tolist())
    oflags = int(np.bitwise_or.reduce(o["seq_flags"])) if B else 0
    print(f"\n{tag}: B={B} mean accepted {acc.mean():.2f} exempt={exempt} hard={hard} flags gpu={fl} oracle={oflags}")
    assert hard == 0, (tag, first)
    if exempt == 0:
        assert fl == oflags, (tag, fl, oflags)
    return acc, fl


@pytest.mark.parametrize("B,n,V,shape,f32", [(48, 12, 5003, "random", False), (33, 25, 4096, "topk", False),
                                             (20, 8, 1, "random", False), (17, 0, 999, "random", False),
                                             (40, 30, 2000, "random", True), (9, 64, 257, "random", False),
                                             (64, 25, 20000, "topk", True), (31, 18, 2001, "random", True)])
def test_trees_against_oracle(oracle, B, n, V, shape, f32):
    d = synth.make_tree_sample(300 + B + n, device=DEV, B=B, n=n, V=V, shape=shape, ragged=True,
                               temps=(0.0, 0.7, 1.0), dtype=torch.float32 if f32 else torch.bfloat16)
    _compare(oracle, d, _rounds(d), tag=(B, n, V, shape, f32))


@pytest.mark.parametrize("max_rounds", [0, 1, 2])
def test_round_limit_truncates_like_the_oracle(oracle, max_rounds):
    d = synth.make_tree_sample(400 + max_rounds, device=DEV, B=64, n=20, V=6007, shape="random",
                               temps=(0.7, 1.0), sigma=2.0)
    d["uniforms"][:, :20] = torch.sqrt(d["uniforms"][:, :20])    # more rejections, so limits bite
    assert _rounds(d) > max_rounds
    _, fl = _compare(oracle, d, max_rounds, tag=f"max_rounds={max_rounds}")
    assert fl & sv.SV_FLAG_TREE_TRUNCATED


def test_enough_rounds_never_truncate(oracle):
    d = synth.make_tree_sample(410, device=DEV, B=64, n=20, V=6007, shape="random", temps=(0.7,), sigma=2.0)
    R = _rounds(d)
    _, fl = _compare(oracle, d, R + 3, oracle_rounds=None, tag="rounds to spare")
    assert not fl & sv.SV_FLAG_TREE_TRUNCATED


def test_default_rounds_from_the_trees(oracle):
    """max_rounds=None: the binding takes the largest need over the batch's
    trees (each cut to its draft length), so no walk is truncated."""
    d = synth.make_tree_sample(420, device=DEV, B=40, n=16, V=4001, shape="random", ragged=True, temps=(0.7, 1.0),
                               sigma=2.0)
    fl = torch.zeros(1, dtype=torch.int32, device=DEV)
    acc, emi, path = sv.spec_verify_tree_sample(d["target"], d["draft"], d["draft_tokens"], d["draft_parents"],
                                                d["draft_lens"], d["temperature"], d["uniforms"], None, err_flags=fl)
    torch.cuda.synchronize()
    o = _oracle(oracle, d)
    assert not int(fl.item()) & sv.SV_FLAG_TREE_TRUNCATED
    same = (acc.cpu().numpy() == o["accepted_len"]) & (emi.cpu().numpy() == o["emitted"]).all(1)
    tie = (o["accept_margin"] < TOL).any(1) | (o["draw_margin"] < TOL)
    assert (same | tie).all()


def test_topk_tree_full_size(oracle):
    """64 sequences, the 26-node top-k tree, V = 128256 bf16, T = 0.7."""
    d = synth.make_tree_sample(7, device=DEV, B=64, n=25, V=128256)
    R = _rounds(d)
    assert R == 3
    acc, _ = _compare(oracle, d, R, tag="full size")
    assert acc.max() >= 2


def test_chain_tree_equals_linear_call():
    d = synth.make(2, 41, device=DEV, B=64, V=9001)
    B, n = d["B"], d["n"]
    chain = torch.arange(n, dtype=torch.int32, device=DEV).repeat(B, 1).contiguous()
    acc, emi, path = sv.spec_verify_tree_sample(d["target"], d["draft"], d["draft_tokens"], chain, d["draft_lens"],
                                                d["temperature"], d["uniforms"], 0)
    acc2, emi2 = sv.spec_verify_sample(d["target"], d["draft"], d["draft_tokens"], d["draft_lens"],
                                       d["temperature"], d["uniforms"])
    torch.cuda.synchronize()
    assert torch.equal(acc, acc2) and torch.equal(emi, emi2)
    for b in range(B):
        k = int(acc[b])
        assert path[b, :k].tolist() == list(range(1, k + 1)) and (path[b, k:] == -1).all()


def test_law_on_the_gpu(oracle):
    """The two-level law case (V = 8, 3 candidates at the root, 2 below each,
    rows that depend on the token prefix), 2 * 10^5 trials in one call: the GPU
    agrees with the oracle trial by trial."""
    h = synth.make_tree_law_case(5, 200_000, device=DEV)
    d = dict(target=h["target"], draft=h["draft"], draft_tokens=h["draft_tokens"], draft_parents=h["draft_parents"],
             draft_lens=h["draft_lens"], temperature=h["temperature"], uniforms=h["uniforms"])
    _compare(oracle, d, sv.sv_tree_rounds(h["draft_parents"][0].tolist()), tag="law case")


@pytest.mark.parametrize("max_rounds", [63, 20])
def test_star_tree_many_rounds(oracle, max_rounds):
    """A star: 64 candidates below the root, so a walk can reject up to 63 of
    them before the last, each later test needing one more round; with 20
    rounds the walks that reject 21 times are truncated like the oracle's."""
    B, n, V = 16, 64, 500
    d = synth.make_tree_sample(440, device=DEV, B=B, n=n, V=V, shape="random", temps=(1.0,), sigma=3.0)
    d["draft_parents"].zero_()
    d["draft_lens"].fill_(n)
    # the candidates are independent draws from the draft at the root
    g = torch.Generator(device=DEV).manual_seed(441)
    gum = -torch.log(-torch.log(torch.rand((B, n, V), generator=g, device=DEV).clamp_(1e-12, 1 - 1e-7)))
    d["draft_tokens"].copy_(torch.argmax(d["draft"][:, :1].float() + gum, dim=-1).to(torch.int32))
    d["uniforms"][:, :n] = 1.0 - (1.0 - d["uniforms"][:, :n]) ** 4     # mostly rejections
    assert sv.sv_tree_rounds([0] * n) == 63
    acc, fl = _compare(oracle, d, max_rounds, tag=f"star, {max_rounds} rounds")
    if max_rounds < 63:
        assert fl & sv.SV_FLAG_TREE_TRUNCATED


@pytest.mark.parametrize("T", [1e-3, 100.0])
def test_extreme_temperatures(oracle, T):
    d = synth.make_tree_sample(450, device=DEV, B=32, n=12, V=3001, shape="random", temps=(T,))
    _compare(oracle, d, _rounds(d), tag=f"T={T}")


def test_masked_vocabulary(oracle):
    """Rows with -inf entries (a masked vocabulary): target and draft rows mask
    different random subsets, so drafted tokens can have p = 0 (never accepted)
    or q = 0 (accepted whenever p > 0), and residuals skip masked entries."""
    d = synth.make_tree_sample(430, device=DEV, B=48, n=14, V=3001, shape="random", ragged=True,
                               temps=(0.0, 0.7, 1.0), dtype=torch.float32)
    g = torch.Generator(device=DEV).manual_seed(431)
    for key, frac in (("target", 0.3), ("draft", 0.3)):
        m = torch.rand(d[key].shape, generator=g, device=DEV) < frac
        d[key].masked_fill_(m, float("-inf"))
    # every row keeps at least one finite entry
    d["target"][..., 0] = 0.0
    d["draft"][..., 0] = 0.0
    acc, fl = _compare(oracle, d, _rounds(d), tag="masked vocabulary")
    assert acc.max() >= 1


def test_law_three_levels_on_the_gpu(oracle):
    """The three-level law case (V = 4, binary tree of 14 candidates), 2 * 10^5
    trials in one call, against the oracle trial by trial."""
    h = synth.make_tree_law_case3(6, 200_000, device=DEV)
    d = dict(target=h["target"], draft=h["draft"], draft_tokens=h["draft_tokens"], draft_parents=h["draft_parents"],
             draft_lens=h["draft_lens"], temperature=h["temperature"], uniforms=h["uniforms"])
    _compare(oracle, d, sv.sv_tree_rounds(h["draft_parents"][0].tolist()), tag="three-level law case")


def test_bad_parents_tokens_and_lengths(oracle):
    d = synth.make_tree_sample(21, device=DEV, B=6, n=5, V=700, shape="random", temps=(0.8,))
    par = d["draft_parents"]
    par[0, 2] = 4                  # not an earlier node
    par[1, 0] = -1
    d["draft_tokens"][2, 0] = 700  # out of range
    d["draft_tokens"][3, 1] = -5
    d["draft_lens"][4] = 9         # clamped
    d["uniforms"][5, 0] = float("nan")
    _, fl = _compare(oracle, d, 4, tag="bad values")
    want = sv.SV_FLAG_BAD_PARENT | sv.SV_FLAG_TOKEN_OOR | sv.SV_FLAG_LEN_CLAMPED | sv.SV_FLAG_BAD_UNIFORM
    assert fl & want == want, fl


def test_workspace_left_zero(oracle):
    ws = torch.zeros(sv.sv_workspace_bytes(64, 25, 40000, sv.SV_BF16), dtype=torch.uint8, device=DEV)
    for seed, (B, n, V, R) in enumerate([(64, 25, 40000, 1), (10, 5, 3001, 4), (64, 25, 40000, 0), (30, 20, 9000, 9)]):
        d = synth.make_tree_sample(500 + seed, device=DEV, B=B, n=n, V=V, shape="random", ragged=True,
                                   temps=(0.0, 0.7))
        _compare(oracle, d, R, ws=ws, tag=f"shared workspace {seed}")
        assert int(ws.count_nonzero()) == 0  # walks, row blocks, counters and sums all cleared


def test_confident_rows_take_the_near_form(oracle):
    """Star trees of 8 candidates at the root whose rows put about 99.9% on one
    shared top token (same logit in both rows) and differ by N(0, 0.3^2) on every
    other token, T = 1: the candidates are the tail tokens the draft favours most,
    so most walks reject several of them and every residual after the first has
    a mass near 1e-4 or below.  The walks' bounds mark those rounds and draws for
    the near form's chunk sums; outputs against the oracle, walk by walk."""
    B, n, V, T = 48, 8, 8192, 1.0
    d = synth.make_tree_sample(460, device=DEV, B=B, n=n, V=V, shape="random", temps=(T,))
    g = torch.Generator(device=DEV).manual_seed(461)
    zt = 3.0 * torch.randn((B, n + 1, V), device=DEV, generator=g)
    top = torch.randint(0, V, (B,), device=DEV, generator=g)
    ar = torch.arange(B, device=DEV)
    zt[ar, 0, top] = zt[:, 0].max(dim=1).values + 9.0
    zd = zt[:, :n].clone() + 0.3 * torch.randn((B, n, V), device=DEV, generator=g)
    zd[ar, 0, top] = zt[ar, 0, top]
    d["target"] = zt.to(d["target"].dtype).contiguous()
    d["draft"] = zd.to(d["draft"].dtype).contiguous()
    t0 = d["target"][:, 0].float()
    q0 = d["draft"][:, 0].float()
    rel = (q0 - q0.max(dim=1, keepdim=True).values) - (t0 - t0.max(dim=1, keepdim=True).values)
    rel[ar, top] = -1e9
    d["draft_tokens"].copy_(torch.topk(rel, n, dim=1).indices.to(torch.int32))
    d["draft_parents"].zero_()
    d["parents_host"] = np.zeros((B, n), np.int32)
    d["draft_lens"].fill_(n)
    d["uniforms"][:, :n] = (1.0 - (1.0 - d["uniforms"][:, :n]) ** 8).clamp_(max=1.0 - 2.0 ** -24)  # mostly rejections
    acc, fl = _compare(oracle, d, _rounds(d), tag="confident rows")
    assert fl == 0


@pytest.mark.parametrize("T", [1e-5, 1e-4, 0.002, 0.005, 0.01, 0.02])
@pytest.mark.parametrize("V", [5814, 6144])
def test_repeated_rejections_at_low_temperature(oracle, T, V):
    """Drafts that are the target plus N(0, 0.003^2) in bf16 (most tokens keep
    the target's logit, the top token among them), tokens drawn from the
    draft's own rows (at low T mostly its top token, so siblings repeat), and
    uniforms pushed towards 1 (mostly rejections): after two or more
    rejections at a node the weight of the tokens the rows share is a product
    of two tails set against first-order terms, which the walk carries as
    kappa = S_d / S_t - lam.  Outputs against the oracle, walk by walk; V = 5814
    takes the element-wise loads."""
    B, n = 64, 12
    seed = 900 + int(T * 1e6) + V
    d = synth.make_tree_sample(seed, device=DEV, B=B, n=n, V=V, shape="random", temps=(T,))
    g = torch.Generator(device=DEV).manual_seed(seed + 1)
    d["draft"] = (d["target"][:, :n].float() + 0.003 * torch.randn((B, n, V), generator=g, device=DEV)).to(
        d["draft"].dtype).contiguous()
    d["uniforms"][:, :n] = (1.0 - (1.0 - d["uniforms"][:, :n]) ** 6).clamp_(max=1.0 - 2.0 ** -24)
    _compare(oracle, d, _rounds(d), tag=f"repeated rejections T={T} V={V}")


@pytest.mark.parametrize("embed", [False, True])
def test_six_token_trees_at_low_temperature(oracle, embed):
    """The six-token trees the oracle is pinned on against exact arithmetic
    (rows sharing their top token, repeated and distinct siblings, T from 0.003
    to 1), bare (element-wise loads) and embedded in 4096-token rows whose
    other entries are -inf in both rows (16-byte loads)."""
    import importlib.util, os
    spec = importlib.util.spec_from_file_location(
        "tree_exact", os.path.join(os.path.dirname(__file__), "test_oracle_tree_exact.py"))
    te = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(te)
    rng = np.random.default_rng(20261203)
    temps = [0.003, 0.01, 0.03, 0.1, 1.0]
    cases = [te._case(rng) for _ in range(300)]
    zt = np.stack([c[0] for c in cases])
    zd = np.stack([c[1] for c in cases])
    x = np.stack([c[2] for c in cases])
    par = np.stack([c[3] for c in cases])
    B, n = x.shape
    temp = np.array([temps[i % len(temps)] for i in range(B)], np.float32)
    u = rng.random((B, n + 1)).astype(np.float32)
    if embed:
        where = np.array([5, 700, 1501, 2048, 3333, 4095])
        big_t = np.full((B, n + 1, 4096), -np.inf, np.float32)
        big_d = np.full((B, n, 4096), -np.inf, np.float32)
        big_t[..., where] = zt
        big_d[..., where] = zd
        zt, zd, x = big_t, big_d, where[x].astype(np.int32)
    d = {"target": torch.as_tensor(zt, device=DEV).to(torch.bfloat16).contiguous(),
         "draft": torch.as_tensor(zd, device=DEV).to(torch.bfloat16).contiguous(),
         "draft_tokens": torch.as_tensor(x, device=DEV), "draft_parents": torch.as_tensor(par, device=DEV),
         "parents_host": par, "draft_lens": torch.full((B,), n, dtype=torch.int32, device=DEV),
         "temperature": torch.as_tensor(temp, device=DEV), "uniforms": torch.as_tensor(u, device=DEV)}
    _compare(oracle, d, _rounds(d), tag=f"six-token trees embed={embed}")


@pytest.mark.parametrize("V", [4096, 4099])
def test_later_sibling_far_below_both_maxima(oracle, V):
    """The oracle's closed form with the rows embedded in V tokens (-5 below
    the top elsewhere): the later sibling's p and q are ~e^-200, far below the
    binary32 range of the far form's terms, and its ratio is exactly 3
    (S_d / S_t = 3, M_1 = 2/3), so it is accepted at every uniform; the
    accepted node's bonus token follows."""
    B = 8
    zt = np.full((B, 3, V), -5.0, np.float32)
    zd = np.full((B, 2, V), -5.0, np.float32)
    zt[:, 0, 100] = 0.0
    zt[:, 0, V - 3] = -2.0
    zd[:, 0, [100, 2000, V - 1]] = 0.0
    zd[:, 0, V - 3] = -2.0
    zt[:, 2, 7] = 0.0
    x = np.array([[2000, V - 3]] * B, np.int32)
    par = np.zeros((B, 2), np.int32)
    u = np.random.default_rng(5).random((B, 3)).astype(np.float32)
    t = lambda a: torch.as_tensor(a, device=DEV)
    d = {"target": t(zt).to(torch.bfloat16).contiguous(), "draft": t(zd).to(torch.bfloat16).contiguous(),
         "draft_tokens": t(x), "draft_parents": t(par), "parents_host": par,
         "draft_lens": torch.full((B,), 2, dtype=torch.int32, device=DEV),
         "temperature": torch.full((B,), 0.01, dtype=torch.float32, device=DEV), "uniforms": t(u)}
    acc, emi, path, fl = _run(d, _rounds(d))
    assert acc.tolist() == [1] * B, acc
    assert emi[:, :3].tolist() == [[V - 3, 7, -1]] * B, emi
    _compare(oracle, d, _rounds(d), tag=f"deep later sibling V={V}")


@pytest.mark.parametrize("same_tile", [True, False])
@pytest.mark.parametrize("T", [1.3e-6, 1e-5, 0.7])
def test_leaf_draw_among_tied_maxima(oracle, same_tile, T):
    """A walk that accepts the root's only child draws from the leaf's target
    row alone.  That row holds three tokens tied at its maximum 15.375 (next
    value 15.0625); at T = 1.3e-6, m c passes 2^24, where the far form's units
    2^(z c - fl(m c)) and the target's 2^((z - m) c) differ by up to a factor
    2, so the draw must scan the picked tile in the units of its tile sums.
    The tie splits the draw in thirds: uniforms in each third pick the first,
    second and third tied token in index order (ties in one tile, or in three)."""
    V = 3344
    ties = [89, 1038, 1413] if same_tile else [89, 2100, 3300]
    us = [0.1, 0.4, 0.7, 0.95, 0.34, 0.66]
    B = len(us)
    g = np.random.default_rng(3)
    zt = np.round((13.0 + g.random((B, 2, V))) * 16.0) / 16.0  # values below the tie, bf16-exact
    zt[:, 1, ties] = 15.375
    zt[:, 1, 7] = 15.0625
    zt = zt.astype(np.float32)
    zd = zt[:, :1].copy()                                        # draft = target at the root: accepted
    x = np.full((B, 1), 500, np.int32)
    par = np.zeros((B, 1), np.int32)
    u = np.zeros((B, 2), np.float32)
    u[:, 0] = 0.5
    u[:, 1] = us
    t = lambda a: torch.as_tensor(a, device=DEV)
    d = {"target": t(zt).to(torch.bfloat16).contiguous(), "draft": t(zd).to(torch.bfloat16).contiguous(),
         "draft_tokens": t(x), "draft_parents": t(par), "parents_host": par,
         "draft_lens": torch.ones(B, dtype=torch.int32, device=DEV),
         "temperature": torch.full((B,), T, dtype=torch.float32, device=DEV), "uniforms": t(u)}
    acc, emi, path, fl = _run(d, _rounds(d))
    assert acc.tolist() == [1] * B, acc
    if T < 1e-4:
        want = [ties[min(int(uu * 3), 2)] for uu in us]
        assert emi[:, 1].tolist() == want, (emi[:, 1].tolist(), want)
    _compare(oracle, d, _rounds(d), tag=f"leaf draw T={T} same_tile={same_tile}")


@pytest.mark.parametrize("T", [1e-5, 1e-3, 0.7])
def test_masked_rows_at_low_temperature(oracle, T):
    """Sampling trees whose rows mask tokens (-inf) in both rows, in the draft
    only (q(x) = 0: a drafted token there is accepted) or in the target only
    (p(x) = 0: rejected), drafts close to the target (most tokens share their
    relative logits), uniforms pushed towards rejection: outputs against the
    oracle, walk by walk."""
    B, n, V = 48, 12, 6144
    seed = 1700 + int(T * 1e5)
    d = synth.make_tree_sample(seed, device=DEV, B=B, n=n, V=V, shape="random", temps=(T,))
    g = torch.Generator(device=DEV).manual_seed(seed + 1)
    d["draft"] = (d["target"][:, :n].float() + 0.01 * torch.randn((B, n, V), generator=g, device=DEV)).to(
        d["draft"].dtype)
    for which, frac in (("both", 0.3), ("draft", 0.05), ("target", 0.05)):
        m = torch.rand((B, 1, V), generator=g, device=DEV) < frac
        if which in ("both", "target"):
            d["target"] = d["target"].masked_fill(m, float("-inf"))
        if which in ("both", "draft"):
            d["draft"] = d["draft"].masked_fill(m, float("-inf"))
    d["target"] = d["target"].contiguous()
    d["draft"] = d["draft"].contiguous()
    d["uniforms"][:, :n] = (1.0 - (1.0 - d["uniforms"][:, :n]) ** 6).clamp_(max=1.0 - 2.0 ** -24)
    _compare(oracle, d, _rounds(d), tag=f"masked rows T={T}")
