"""GPU parity of the fused logit projection + greedy verify
(spec_verify_greedy_lmhead) and of the projection kernel itself
(sv_lmhead_logits_debug), against the oracle's double-precision projection and
its greedy rule.

Two input recipes (draft_token_verification_08_amd.synth.make_lmhead):
  exact     every partial sum of every logit is exactly representable in
            binary32, so the logits are the same in any summation order: the
            projection must equal the oracle bit for bit and every decision must
            match, ties (duplicated weight rows) included, with no exemption;
  gaussian  bf16 normals: each logit may differ from the exact value by at most
            the binary32 summation bound 2 * gamma_H * sum_k |h_k w_k|
            (gamma_H = H u / (1 - H u), u = 2^-24; the factor 2 leaves room for
            the matrix cores' internal rounding).  Decisions must match except in
            sequences holding a row whose top two distinct exact logits are
            closer than twice that bound; those are checked for validity."""
import numpy as np
import pytest
import torch

import draft_token_verification_08_amd as sv
from draft_token_verification_08_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _host(d):
    H = d["H"]
    return synth.bf16_bits(d["hidden"]).reshape(-1, H), synth.bf16_bits(d["weight"])


def _oracle_greedy(oracle, d, seqs=None, threads=16):
    """The oracle's decisions for the sequences `seqs` (all when None) from its
    own double-precision logits; returns (result dict, logits [b, n+1, V])."""
    B, n, V = d["B"], d["n"], d["V"]
    h, w = _host(d)
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    rows = (seqs[:, None] * (n + 1) + np.arange(n + 1)[None, :]).reshape(-1).astype(np.int32)
    z = oracle.lmhead_logits(h, w, rows=rows, threads=threads).reshape(len(seqs), n + 1, V)
    r = oracle.verify_greedy(z, d["draft_tokens"].cpu().numpy()[seqs], d["draft_lens"].cpu().numpy()[seqs],
                             threads=threads)
    return r, z


def _run(d, **kw):
    acc, emi = sv.spec_verify_greedy_lmhead(d["hidden"], d["weight"], d["draft_tokens"], d["draft_lens"], **kw)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), emi.cpu().numpy()


@pytest.mark.parametrize("B,n,V,H,seed", [(9, 4, 1000, 192, 0), (26, 4, 257, 64, 1), (52, 4, 4096, 512, 2),
                                          (3, 0, 300, 128, 3), (2, 1, 1, 64, 4), (1, 0, 33, 64, 5)])
def test_projection_bit_exact_on_exact_inputs(oracle, B, n, V, H, seed):
    """Several row and vocabulary tiles with ragged tails (M = B*(n+1) and V not
    multiples of the 256 x 256 tile)."""
    d = synth.make_lmhead(100 + seed, device=DEV, B=B, n=n, V=V, H=H)
    got = sv.sv_lmhead_logits_debug(d["hidden"], d["weight"])
    torch.cuda.synchronize()
    h, w = _host(d)
    ref = oracle.lmhead_logits(h, w, threads=16)
    assert np.array_equal(got.cpu().numpy().astype(np.float64), ref)


def test_projection_within_summation_bound_on_gaussian_inputs(oracle):
    d = synth.make_lmhead(110, device=DEV, B=20, n=4, V=3000, H=1024, exact=False)
    got = sv.sv_lmhead_logits_debug(d["hidden"], d["weight"]).cpu().numpy().astype(np.float64)
    h, w = _host(d)
    ref = oracle.lmhead_logits(h, w, threads=16)
    hf = d["hidden"].reshape(-1, 1024).double().cpu().numpy()
    wf = d["weight"].double().cpu().numpy()
    H, u = 1024, 2.0 ** -24
    bound = 2 * (H * u / (1 - H * u)) * (np.abs(hf) @ np.abs(wf).T)
    err = np.abs(got - ref)
    assert (err <= bound).all(), (err / np.maximum(bound, 1e-300)).max()


@pytest.mark.parametrize("B,n,V,H,ragged,seed", [(37, 4, 5003, 256, False, 0), (64, 4, 2048, 128, True, 1),
                                                 (24, 8, 1001, 320, True, 2), (130, 1, 700, 64, False, 3),
                                                 (5, 2, 1, 64, True, 4), (9, 3, 7, 128, True, 5)])
def test_greedy_lmhead_exact(oracle, B, n, V, H, ragged, seed):
    d = synth.make_lmhead(200 + seed, device=DEV, B=B, n=n, V=V, H=H, ragged=ragged)
    fl = torch.zeros(1, dtype=torch.int32, device=DEV)
    acc, emi = _run(d, err_flags=fl)
    r, _ = _oracle_greedy(oracle, d)
    assert np.array_equal(acc, r["accepted_len"])
    assert np.array_equal(emi, r["emitted"])
    assert int(fl.item()) == int(np.bitwise_or.reduce(r["seq_flags"]))


def test_greedy_lmhead_full_config(oracle):
    """B=256, n=4, V=128256, H=8192 (Llama-70B-sized projection, 2.1 GB of
    weight): every decision of a sample of 24 sequences, bit-exact."""
    d = synth.make_lmhead(303, device=DEV)
    acc, emi = _run(d)
    seqs = np.sort(np.random.default_rng(3).choice(d["B"], size=24, replace=False))
    r, _ = _oracle_greedy(oracle, d, seqs)
    assert np.array_equal(acc[seqs], r["accepted_len"])
    assert np.array_equal(emi[seqs], r["emitted"])
    # the recipe makes most drafts match: the decisions are not trivially all-reject
    assert acc.mean() > 0.5


def test_greedy_lmhead_single_token_mtp_shape(oracle):
    """The single-token MTP workload's projection shape (DeepSeek R1: D=512, n=1,
    V=129280, H=7168, 1024 rows): a sample of 32 sequences, bit-exact, with the
    MTP token shift/insert and hidden carry."""
    d = synth.make_lmhead(304, device=DEV, B=512, n=1, V=129280, H=7168, ragged=True)
    tok = d["tokens"].clone()
    dst = torch.empty_like(d["hidden"])
    acc, emi = _run(d, tokens=tok, hidden_dst=dst)
    seqs = np.sort(np.random.default_rng(4).choice(d["B"], size=32, replace=False))
    r, _ = _oracle_greedy(oracle, d, seqs)
    assert np.array_equal(acc[seqs], r["accepted_len"])
    assert np.array_equal(emi[seqs], r["emitted"])
    ref_tok, _ = oracle.mtp_shift_insert(d["tokens"].cpu().numpy(), None, acc, emi)
    assert np.array_equal(tok.cpu().numpy(), ref_tok)
    assert torch.equal(dst.view(torch.int16), d["hidden"].view(torch.int16))


def _gap_and_bound(d, z, seqs):
    """Per row (of the chosen sequences): the distance from the top exact logit
    to the next smaller one, and the binary32 bound 2 gamma_H max_v sum |h w|."""
    n, H = d["n"], d["H"]
    s = np.sort(z, axis=-1)
    top = s[..., -1:]
    below = np.where(s < top, s, -np.inf).max(axis=-1)
    gap = top[..., 0] - below
    hf = d["hidden"].double().cpu().numpy()[seqs].reshape(-1, H)
    wf = d["weight"].double().cpu().numpy()
    u = 2.0 ** -24
    bound = 2 * (H * u / (1 - H * u)) * (np.abs(hf) @ np.abs(wf).T).max(axis=1)
    return gap, bound.reshape(len(seqs), n + 1)


def test_greedy_lmhead_gaussian(oracle):
    d = synth.make_lmhead(400, device=DEV, B=48, n=4, V=20000, H=1024, exact=False, ragged=True)
    acc, emi = _run(d)
    seqs = np.arange(d["B"])
    r, z = _oracle_greedy(oracle, d, seqs)
    gap, bound = _gap_and_bound(d, z, seqs)
    x = d["draft_tokens"].cpu().numpy()
    lens = d["draft_lens"].cpu().numpy()
    exempt = 0
    for b in seqs:
        if acc[b] == r["accepted_len"][b] and np.array_equal(emi[b], r["emitted"][b]):
            continue
        L = lens[b]
        near = (gap[b, :L + 1] <= 2 * bound[b, :L + 1]).any()
        assert near, (b, acc[b], r["accepted_len"][b], gap[b], bound[b])
        exempt += 1
        # validity: every accepted draft and the emitted token are within the bound of the row's top
        k = acc[b]
        for j in range(k):
            assert z[b, j, x[b, j]] >= z[b, j].max() - 2 * bound[b, j]
        assert z[b, k, emi[b, k]] >= z[b, k].max() - 2 * bound[b, k]
    assert exempt <= 2, exempt


def test_greedy_lmhead_mtp_and_workspace(oracle):
    """The MTP token shift/insert and the hidden-state carry inside the fused
    call equal the oracle's shift/insert applied to the decisions; a second call
    on the same workspace gives the same result and leaves it zero."""
    B, n, V, H = 40, 4, 3000, 192
    d = synth.make_lmhead(500, device=DEV, B=B, n=n, V=V, H=H, ragged=True)
    need = sv.sv_workspace_bytes(B, n, V, sv.SV_BF16)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    r, _ = _oracle_greedy(oracle, d)
    for _ in range(2):
        tok = d["tokens"].clone()
        dst = torch.zeros_like(d["hidden"])
        acc, emi = _run(d, tokens=tok, hidden_dst=dst, workspace=ws)
        assert np.array_equal(acc, r["accepted_len"]) and np.array_equal(emi, r["emitted"])
        ref_tok, ref_hid = oracle.mtp_shift_insert(d["tokens"].cpu().numpy(),
                                                   d["hidden"].cpu().view(torch.int16).numpy(), acc, emi)
        assert np.array_equal(tok.cpu().numpy(), ref_tok)
        assert np.array_equal(dst.cpu().view(torch.int16).numpy(), ref_hid)
    assert int(ws.count_nonzero()) == 0
    # hidden_dst == hidden: nothing copied, tokens still shifted
    tok = d["tokens"].clone()
    before = d["hidden"].clone()
    acc, emi = _run(d, tokens=tok, hidden_dst=d["hidden"])
    assert torch.equal(d["hidden"].view(torch.int16), before.view(torch.int16))
    ref_tok, _ = oracle.mtp_shift_insert(d["tokens"].cpu().numpy(), None, acc, emi)
    assert np.array_equal(tok.cpu().numpy(), ref_tok)


def test_greedy_lmhead_bad_tokens_and_lengths(oracle):
    """Out-of-range drafts are rejected at their slot and flagged; lengths
    outside [0, n] are clamped and flagged, as in the oracle."""
    B, n, V, H = 12, 4, 900, 128
    d = synth.make_lmhead(600, device=DEV, B=B, n=n, V=V, H=H)
    d["draft_tokens"][0, 1] = V
    d["draft_tokens"][1, 0] = -3
    d["draft_lens"][2] = n + 3
    d["draft_lens"][3] = -1
    fl = torch.zeros(1, dtype=torch.int32, device=DEV)
    acc, emi = _run(d, err_flags=fl)
    r, _ = _oracle_greedy(oracle, d)
    assert np.array_equal(acc, r["accepted_len"]) and np.array_equal(emi, r["emitted"])
    assert int(fl.item()) == int(np.bitwise_or.reduce(r["seq_flags"]))
    assert int(fl.item()) & (sv.SV_FLAG_TOKEN_OOR | sv.SV_FLAG_LEN_CLAMPED) == \
        (sv.SV_FLAG_TOKEN_OOR | sv.SV_FLAG_LEN_CLAMPED)


def test_fused_equals_projection_then_greedy_verify():
    """The two library paths agree: the projection's logits fed to
    spec_verify_greedy give the fused call's decisions (exact inputs)."""
    d = synth.make_lmhead(700, device=DEV, B=32, n=4, V=6000, H=256, ragged=True)
    acc, emi = _run(d)
    z = sv.sv_lmhead_logits_debug(d["hidden"], d["weight"]).view(32, 5, 6000)
    a2, e2 = sv.spec_verify_greedy(z, d["draft_tokens"], d["draft_lens"])
    torch.cuda.synchronize()
    assert np.array_equal(acc, a2.cpu().numpy()) and np.array_equal(emi, e2.cpu().numpy())


def test_random_shapes_against_oracle(oracle):
    """Twelve seeded random shapes (B, n, V, H with H a multiple of 64, V and
    B*(n+1) mostly not multiples of the tile, n = 0 included): every decision and
    every flag equal the oracle's on exact-sum inputs."""
    rng = np.random.default_rng(2024)
    for case in range(12):
        B = int(rng.integers(1, 70))
        n = int(rng.integers(0, 9))
        V = int(rng.integers(1, 3000))
        H = 64 * int(rng.integers(1, 9))
        d = synth.make_lmhead(900 + case, device=DEV, B=B, n=n, V=V, H=H, ragged=True)
        fl = torch.zeros(1, dtype=torch.int32, device=DEV)
        acc, emi = _run(d, err_flags=fl)
        r, _ = _oracle_greedy(oracle, d)
        assert np.array_equal(acc, r["accepted_len"]), (case, B, n, V, H)
        assert np.array_equal(emi, r["emitted"]), (case, B, n, V, H)
        assert int(fl.item()) == int(np.bitwise_or.reduce(r["seq_flags"])), (case, B, n, V, H)
