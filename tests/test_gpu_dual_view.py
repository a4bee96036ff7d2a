"""GPU parity of dv_dual_view_attention (COVER's dual-view attention) against
oracle.dual_view. Tolerance from the arithmetic: bf16 inputs are exact in both,
products accumulate in fp32, and the probabilities are rounded to bf16 for the
second product, which moves an output by at most 2^-9 of the largest value
magnitude; the test allows 4e-3 of it (plus 4e-3 relative)."""

import numpy as np
import pytest
import torch

import token_verification_row_amd as dv
import workloads as W
from oracle import dual_view as ODV

pytestmark = pytest.mark.gpu


def _dev():
    return torch.device("cuda:0")


def _bf16(x, dev):
    bits = W.round_bf16_bits(x.astype(np.float32))
    return bits, torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)


def _widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _case(B, H, Hkv, L, D, p_seed, seed):
    rng = np.random.default_rng(seed)
    dev = _dev()
    shapes = {"q": (B, H, L, D), "kc": (B, Hkv, L, D), "vc": (B, Hkv, L, D), "kp": (B, Hkv, L, D), "vp": (B, Hkv, L, D)}
    host, gpu = {}, {}
    for k, shp in shapes.items():
        host[k], gpu[k] = _bf16(rng.standard_normal(shp), dev)
    sd = (rng.random((B, L)) < p_seed).astype(np.uint8)
    return host, gpu, sd, torch.from_numpy(sd).to(dev)


def _check(host, gpu, sd, gsd, scale, ctx):
    out = dv.dv_dual_view_attention(gpu["q"], gpu["kc"], gpu["vc"], gpu["kp"], gpu["vp"], gsd, scale=scale)
    ref = ODV.dual_view_attention(_widen(host["q"]), _widen(host["kc"]), _widen(host["vc"]), _widen(host["kp"]),
                                  _widen(host["vp"]), sd, scale)
    vmax = max(np.abs(_widen(host["vc"])).max(), np.abs(_widen(host["vp"])).max())
    got = out.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=4e-3, atol=4e-3 * vmax, err_msg=ctx)
    return got, ref


@pytest.mark.parametrize("B,H,Hkv,L,D,p_seed", [(1, 2, 1, 32, 64, 0.3), (1, 4, 2, 96, 128, 0.3),
                                                (2, 4, 4, 256, 128, 0.25), (1, 8, 2, 512, 64, 0.2),
                                                (1, 2, 2, 160, 128, 0.0), (1, 2, 1, 64, 128, 1.0),
                                                (1, 4, 2, 96, 64, 0.3), (2, 4, 2, 160, 64, 0.5),
                                                (1, 3, 1, 224, 64, 1.0), (1, 2, 2, 288, 128, 0.5)])
def test_dual_view_attention(B, H, Hkv, L, D, p_seed):
    print(f"case: dual view B={B} H={H} Hkv={Hkv} L={L} D={D} seeds={p_seed}", flush=True)
    host, gpu, sd, gsd = _case(B, H, Hkv, L, D, p_seed, seed=L + D + H)
    got, ref = _check(host, gpu, sd, gsd, D ** -0.5, f"B={B} H={H} L={L} D={D}")
    if 0 < p_seed < 1:
        # the override matters: plain attention over the current K/V differs
        plain = ODV.dual_view_attention(_widen(host["q"]), _widen(host["kc"]), _widen(host["vc"]),
                                        _widen(host["kp"]), _widen(host["vp"]), np.zeros_like(sd), D ** -0.5)
        assert np.abs(plain - ref).max() > 0.05


def test_leave_one_out_on_gpu():
    """A seed query does not see its own cached K/V; every other query does."""
    print("case: dual view leave-one-out", flush=True)
    host, gpu, sd, gsd = _case(1, 2, 2, 128, 128, 0.0, seed=5)
    sd[0, 37] = 1
    gsd = torch.from_numpy(sd).to(_dev())
    base, _ = _check(host, gpu, sd, gsd, 0.1, "base")
    for name in ("kp", "vp"):
        h2 = dict(host)
        x = _widen(host[name]).astype(np.float32)
        x[:, :, 37] += 4.0
        h2[name], g = _bf16(x, _dev())
        g2 = dict(gpu)
        g2[name] = g
        moved, _ = _check(h2, g2, sd, gsd, 0.1, f"moved {name}")
        # row 37 keeps (up to the bf16 rounding of its own weight), the others move
        np.testing.assert_allclose(moved[:, :, 37], base[:, :, 37], atol=4e-3 * 8)
        assert np.abs(moved[:, :, :37] - base[:, :, :37]).max() > 1e-3


def test_bench_shape_sampled_heads():
    """The shape and launch the benchmark times (32 sequences x 28 heads over 4
    key/value heads, 1024 positions, head_dim 128, 10% seeds), checked on a
    sample of (sequence, head) pairs against the oracle run on those heads."""
    print("case: dual view 32x28x1024x128 sampled heads", flush=True)
    dev = _dev()
    B, H, Hkv, L, D = 32, 28, 4, 1024, 128
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    q = torch.randn((B, H, L, D), generator=g, device=dev).to(torch.bfloat16)
    kv = [torch.randn((B, Hkv, L, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(4)]
    sd = (torch.rand((B, L), generator=g, device=dev) < 0.1).to(torch.uint8)
    out = dv.dv_dual_view_attention(q, *kv, sd, scale=D ** -0.5)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (13, 6), (31, 27), (20, 15)):
        gh = h // (H // Hkv)
        host = lambda t, i: t[b:b + 1, i:i + 1].float().cpu().numpy().astype(np.float64)
        ref = ODV.dual_view_attention(host(q, h), *(host(t, gh) for t in kv), sd[b:b + 1].cpu().numpy(), D ** -0.5)
        vmax = max(float(kv[1][b, gh].float().abs().max()), float(kv[3][b, gh].float().abs().max()))
        got = out[b:b + 1, h:h + 1].cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(got, ref, rtol=4e-3, atol=4e-3 * vmax, err_msg=f"b={b} h={h}")
