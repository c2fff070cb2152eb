"""GPU parity of mla_v_up_proj (W_UV up-projection and sigmoid gate)
against the float64 oracle.

Bar, from the arithmetic: the kernel accumulates 512 bf16 products in
float32 (error ~1e-5 at unit scale), applies the gate in float32 and rounds
once to bf16 (relative 2^-9), so |got - ref| <= 4e-3 |ref| + 1e-4.
"""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from head_latent_attention_sparse_amd import workloads
from head_latent_attention_sparse_amd.workloads import bf16_bits
from oracle import v_up_proj as oracle_v_up_proj
from tests.helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
RTOL, ATOL = 4e-3, 1e-4


def check(got, ref):
    got = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    bad = np.argwhere(err > 0)
    assert bad.size == 0, f"{len(bad)} values off, first {bad[:3].tolist()}, worst excess {err.max():.3g}"


@pytest.mark.parametrize("t,h", [(1, 1), (5, 4), (64, 16), (100, 12), (300, 16), (129, 128)])
@pytest.mark.parametrize("gated", [False, True])
def test_v_up_proj(t, h, gated):
    say(f"v_up_proj T={t} H={h} gate={gated}")
    w = workloads.v_up_proj_inputs(tokens=t, heads=h)
    gate = w.gate.to(DEV) if gated else None
    got = mla.v_up_proj(w.latent.to(DEV), w.w_uv.to(DEV), gate=gate)
    torch.cuda.synchronize()
    check(got, oracle_v_up_proj(bf16_bits(w.latent), bf16_bits(w.w_uv), bf16_bits(w.gate) if gated else None))


def test_v_up_proj_on_forward_output_layout_and_wide_out():
    """latent as the forward's out [T, H, 520] view; out written into a wider buffer."""
    say("v_up_proj strided")
    t, h = 77, 16
    w = workloads.v_up_proj_inputs(tokens=t, heads=h)
    lat = torch.zeros((t, h, 520), dtype=torch.bfloat16, device=DEV)
    lat[:, :, :512] = w.latent.to(DEV)
    gate_wide = torch.zeros((t, h * 128 + 64), dtype=torch.bfloat16, device=DEV)
    gate_wide[:, :h * 128] = w.gate.to(DEV)
    out = torch.full((t, h, 136), -5.0, dtype=torch.bfloat16, device=DEV)
    mla.v_up_proj(lat, w.w_uv.to(DEV), gate=gate_wide[:, :h * 128], out=out[:, :, :128])
    torch.cuda.synchronize()
    check(out[:, :, :128], oracle_v_up_proj(bf16_bits(w.latent), bf16_bits(w.w_uv), bf16_bits(w.gate)))
    assert torch.all(out[:, :, 128:].cpu() == -5.0), "wrote past column 128"


def test_v_up_proj_full():
    say("v_up_proj T=4096 H=16 gated")
    w = workloads.v_up_proj_inputs()
    got = mla.v_up_proj(w.latent.to(DEV), w.w_uv.to(DEV), gate=w.gate.to(DEV))
    torch.cuda.synchronize()
    check(got, oracle_v_up_proj(bf16_bits(w.latent), bf16_bits(w.w_uv), bf16_bits(w.gate)))


def test_v_up_proj_empty_and_rejections():
    say("v_up_proj empty / rejections")
    wuv = torch.zeros((4, 512, 128), dtype=torch.bfloat16, device=DEV)
    assert mla.v_up_proj(torch.zeros((0, 4, 512), dtype=torch.bfloat16, device=DEV), wuv).shape == (0, 4, 128)
    with pytest.raises(ValueError):
        mla.v_up_proj(torch.zeros((3, 4, 512), dtype=torch.bfloat16, device=DEV), wuv[:3])
    with pytest.raises(ValueError):  # rows not 16-byte aligned
        base = torch.zeros((3 * 4 * 516 + 4,), dtype=torch.bfloat16, device=DEV)
        mla.v_up_proj(base[4:].view(3, 4, 516)[:, :, :512], wuv)


@pytest.mark.parametrize("t,h", [(1, 1), (64, 16), (300, 12), (129, 128), (4096, 16)])
@pytest.mark.parametrize("gated", [False, True])
def test_v_up_proj_prepared_weights(t, h, gated):
    """mla_v_up_proj_prepared on mla_v_up_proj_prepare_weights' layout gives
    mla_v_up_proj's results bit for bit (and so meets the oracle's bar), and
    the preparation leaves W_UV untouched."""
    say(f"v_up_proj prepared T={t} H={h} gate={gated}")
    w = workloads.v_up_proj_inputs(tokens=t, heads=h)
    lat, wuv = w.latent.to(DEV), w.w_uv.to(DEV)
    gate = w.gate.to(DEV) if gated else None
    prepared = mla.prepare_w_uv(wuv)
    got = mla.v_up_proj(lat, prepared, gate=gate, prepared=True)
    plain = mla.v_up_proj(lat, wuv, gate=gate)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), plain.view(torch.int16)), "prepared path differs from the plain one"
    assert torch.equal(wuv.cpu(), w.w_uv), "W_UV changed"
    assert not torch.equal(prepared.cpu(), w.w_uv) or h * t == 0, "the prepared layout is a different order"
    if t <= 300:
        check(got, oracle_v_up_proj(bf16_bits(w.latent), bf16_bits(w.w_uv), bf16_bits(w.gate) if gated else None))
