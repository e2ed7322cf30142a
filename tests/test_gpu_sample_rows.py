"""GPU parity of sv_sample_rows (standard sampling of one token from a row the
device chooses) against the oracle, and the workspace zero-fill contract."""
import numpy as np
import pytest
import torch

import draft_token_verification_08_amd as sv
from draft_token_verification_08_amd import synth
from svcompare import TOL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(oracle, z, T, u, ri, tokens, flags):
    zh = synth.host_logits(z)
    o = oracle.sample_rows(zh, T.cpu().numpy(), u.cpu().numpy(), None if ri is None else ri.cpu().numpy(),
                           threads=16)
    got = tokens.cpu().numpy()
    diff = np.nonzero(got != o["tokens"])[0]
    if diff.size:
        # a differing draw is allowed only at a CDF boundary closer than 1e-5 of the mass
        B = z.shape[0]
        idx = ri.cpu().numpy() if ri is not None else np.zeros(B, np.int32)
        rows = zh[np.arange(B), np.clip(idx, 0, z.shape[1] - 1)][:, None, :]
        v = oracle.verify_sample(rows, None, np.zeros((B, 0), np.int32), np.zeros(B, np.int32),
                                 T.cpu().numpy(), u.cpu().numpy().reshape(B, 1), threads=16)
        for b in diff:
            assert float(T[b]) > 0 and v["draw_margin"][b] < TOL, (b, got[b], o["tokens"][b])
    assert flags == int(np.bitwise_or.reduce(o["seq_flags"]))
    return diff.size


@pytest.mark.parametrize("dt,B,R,V", [(torch.bfloat16, 512, 2, 129280), (torch.bfloat16, 256, 5, 128256),
                                       (torch.float32, 33, 3, 1001), (torch.bfloat16, 17, 4, 7)])
def test_carried_logits_at_accepted_slot(oracle, dt, B, R, V):
    """The next step's first draft token from the carried draft logits at slot a_b
    (row_index = accepted lengths produced on the device by a verify step)."""
    g = torch.Generator(device=DEV).manual_seed(B + R)
    z = (3 * torch.randn((B, R, V), generator=g, device=DEV)).to(dt)
    acc = torch.randint(0, R, (B,), generator=g, device=DEV, dtype=torch.int32)
    T = torch.tensor([0.0, 0.6, 1.0], device=DEV)[torch.randint(0, 3, (B,), generator=g, device=DEV)]
    u = torch.rand((B,), generator=g, device=DEV)
    fl = torch.zeros(1, dtype=torch.int32, device=DEV)
    tok = sv.sv_sample_rows(z, T, u, acc, err_flags=fl)
    torch.cuda.synchronize()
    _check(oracle, z, T, u, acc, tok, int(fl.item()))


def test_draft_step_sampling_rows(oracle):
    """The draft's per-step sampling over [B, V] (one row per sequence)."""
    g = torch.Generator(device=DEV).manual_seed(5)
    B, V = 256, 128256
    z = (3 * torch.randn((B, V), generator=g, device=DEV)).to(torch.bfloat16)
    T = torch.full((B,), 0.7, device=DEV)
    T[::5] = 0.0
    u = torch.rand((B,), generator=g, device=DEV)
    tok = sv.sv_sample_rows(z, T, u)
    torch.cuda.synchronize()
    _check(oracle, z.unsqueeze(1), T, u, None, tok, 0)


def test_row_index_clamped_and_flagged(oracle):
    g = torch.Generator(device=DEV).manual_seed(9)
    z = torch.randn((6, 3, 4096), generator=g, device=DEV)
    ri = torch.tensor([-2, 0, 1, 2, 3, 99], dtype=torch.int32, device=DEV)
    T = torch.zeros(6, device=DEV)
    u = torch.zeros(6, device=DEV)
    fl = torch.zeros(1, dtype=torch.int32, device=DEV)
    tok = sv.sv_sample_rows(z, T, u, ri, err_flags=fl)
    torch.cuda.synchronize()
    _check(oracle, z, T, u, ri, tok, int(fl.item()))
    assert int(fl.item()) & sv.SV_FLAG_ROW_CLAMPED


def test_workspace_left_zero_across_shapes():
    """Every completed call leaves the workspace zero-filled, so one workspace
    serves calls of any shape that fits it."""
    ws = sv.Workspace(DEV).get(8 << 20)
    calls = [
        lambda: sv.spec_verify_sample(*[synth.make(5, 1, device=DEV, B=40, V=6007)[k] for k in
                                        ("target", "draft", "draft_tokens", "draft_lens", "temperature",
                                         "uniforms")], workspace=ws),
        lambda: sv.spec_verify_greedy(*[synth.make(3, 2, device=DEV, B=64, V=4096, H=0)[k] for k in
                                        ("target", "draft_tokens", "draft_lens")], workspace=ws),
        lambda: sv.sv_sample_rows((3 * torch.randn((300, 2, 20000), device=DEV)).to(torch.bfloat16),
                                  torch.full((300,), 0.9, device=DEV), torch.rand(300, device=DEV),
                                  torch.randint(0, 2, (300,), device=DEV, dtype=torch.int32), workspace=ws),
        lambda: sv.spec_verify_sample(*[synth.make(2, 3, device=DEV, B=16, V=50000)[k] for k in
                                        ("target", "draft", "draft_tokens", "draft_lens", "temperature",
                                         "uniforms")], workspace=ws),
    ]
    for f in calls:
        f()
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
