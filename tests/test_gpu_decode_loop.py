"""Several greedy decode steps composed on the device, the way a serving loop
chains the entry points (Target-draft section, decode paragraph; Single-token
MTP scheduling section), with no host work between them, checked step by step
against the oracle running the same chain on the CPU:

  1. the draft loop: draft token j is the argmax of draft row j
     (sv_sample_rows, T = 0, row chosen on the device with row_index = j);
  2. the verify step with the MTP token shift/insert and hidden carry
     (spec_verify_greedy_mtp);
  3. the next step's first draft token from the carried draft logits at the
     accepted slot (sv_sample_rows, row_index = accepted_len).

The token buffer each side carries into the next step is its own, so a single
divergence anywhere would propagate; greedy decisions have no exemptions."""
import numpy as np
import pytest
import torch

import draft_token_verification_08_amd as sv
from draft_token_verification_08_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_greedy_decode_loop_matches_oracle(oracle):
    B, n, V, H, steps = 48, 4, 5003, 32, 4
    g = torch.Generator(device=DEV).manual_seed(123)
    tokens = torch.randint(0, V, (B, n + 1), generator=g, device=DEV, dtype=torch.int32)
    tok_o = tokens.cpu().numpy().copy()
    zeros_T = torch.zeros(B, device=DEV)
    u = torch.rand(B, generator=g, device=DEV)
    for step in range(steps):
        zd = (3.0 * torch.randn((B, n + 1, V), generator=g, device=DEV)).to(torch.bfloat16)  # draft/MTP logits
        zt = (zd.float() + 0.3 * torch.randn((B, n + 1, V), generator=g, device=DEV)).to(torch.bfloat16)
        hidden = torch.randn((B, n + 1, H), generator=g, device=DEV).to(torch.bfloat16)
        lens = torch.randint(0, n + 1, (B,), generator=g, device=DEV, dtype=torch.int32)
        dst = torch.empty_like(hidden)
        # 1. draft loop on the device
        x = torch.empty((B, n), dtype=torch.int32, device=DEV)
        for j in range(n):
            row = torch.full((B,), j, dtype=torch.int32, device=DEV)
            x[:, j] = sv.sv_sample_rows(zd, zeros_T, u, row_index=row)
        # 2. verify + MTP
        acc, emi = sv.spec_verify_greedy_mtp(zt, x.contiguous(), lens, tokens, hidden, dst)
        # 3. next first draft token from the carried draft logits at the accepted slot
        nxt = sv.sv_sample_rows(zd, zeros_T, u, row_index=acc)
        torch.cuda.synchronize()

        zd_h, zt_h = synth.host_logits(zd), synth.host_logits(zt)
        xo = np.stack([oracle.sample_rows(zd_h, np.zeros(B, np.float32), u.cpu().numpy(),
                                          row_index=np.full(B, j, np.int32))["tokens"] for j in range(n)], axis=1)
        assert np.array_equal(x.cpu().numpy(), xo), step
        r = oracle.verify_greedy(zt_h[:, :n + 1], xo, lens.cpu().numpy())
        assert np.array_equal(acc.cpu().numpy(), r["accepted_len"]), step
        assert np.array_equal(emi.cpu().numpy(), r["emitted"]), step
        tok_o, hid_o = oracle.mtp_shift_insert(tok_o, hidden.cpu().view(torch.int16).numpy(), r["accepted_len"],
                                               r["emitted"])
        assert np.array_equal(tokens.cpu().numpy(), tok_o), step
        assert np.array_equal(dst.cpu().view(torch.int16).numpy(), hid_o), step
        no = oracle.sample_rows(zd_h, np.zeros(B, np.float32), u.cpu().numpy(), row_index=r["accepted_len"])
        assert np.array_equal(nxt.cpu().numpy(), no["tokens"]), step
        # some drafts are accepted and some rejected, so the chain is exercised
        if step == 0:
            a = acc.cpu().numpy()
            assert (a > 0).any() and (a < lens.cpu().numpy()).any()
