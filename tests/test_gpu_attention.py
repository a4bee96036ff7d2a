"""GPU parity of dv_influence_drift (COVER's d_in and d_out) against
oracle.attention: float results within the float tolerance, bitwise repeatable."""

import numpy as np
import pytest
import torch

import token_verification_row_amd as dv
import workloads as W
from oracle import attention as OA
from oracle import select as OS
from parity_util import ATOL, RTOL

pytestmark = pytest.mark.gpu


def _dev():
    return torch.device("cuda:0")


def _softmax(x):
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _case(B, H, L, dtype, seed, pad=0, pad_bits=None):
    """Random attention maps (peaky softmax rows) as stored: float32 values or bf16 bits, with ld = L + pad."""
    rng = np.random.default_rng(seed)
    p = _softmax(rng.standard_normal((B, H, L, L)).astype(np.float32) * 3.0).astype(np.float32)
    ld = L + pad
    if dtype == "bf16":
        bits = W.round_bf16_bits(p)
        buf = np.zeros((B, H, L, ld), np.uint16)
        if pad_bits is not None:
            buf[..., L:] = pad_bits
        buf[..., :L] = bits
        t = torch.from_numpy(buf.view(np.int16)).to(_dev()).view(torch.bfloat16)
        host = bits
    else:
        buf = np.zeros((B, H, L, ld), np.float32)
        if pad_bits is not None:
            buf[..., L:] = np.uint32(pad_bits).view(np.float32)
        buf[..., :L] = p
        t = torch.from_numpy(buf).to(_dev())
        host = p
    qm = (rng.random((B, L)) < 0.4).astype(np.uint8)
    nc = (rng.random((B, L)) < 0.2).astype(np.uint8)
    return t[..., :L], host, qm, nc


def _widen(host, dtype):
    if dtype == "bf16":
        return (host.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return host.astype(np.float64)


def _check(B, H, L, dtype, seed, pad=0, pad_bits=None):
    t, host, qm, nc = _case(B, H, L, dtype, seed, pad, pad_bits)
    dev = _dev()
    gq, gn = torch.from_numpy(qm).to(dev), torch.from_numpy(nc).to(dev)
    d_in, d_out = dv.dv_influence_drift(t, gq, gn)
    r_in, r_out = OA.influence_drift(_widen(host, dtype), qm, nc)
    np.testing.assert_allclose(d_in.cpu().numpy(), r_in, rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(d_out.cpu().numpy(), r_out, rtol=RTOL, atol=ATOL)
    d_in2, d_out2 = dv.dv_influence_drift(t, gq, gn)
    assert torch.equal(d_in, d_in2) and torch.equal(d_out, d_out2)   # fixed summation order


@pytest.mark.parametrize("B,H,L,dtype,pad", [(1, 1, 1, "fp32", 3), (1, 3, 7, "bf16", 1), (2, 5, 64, "fp32", 0),
                                             (2, 5, 64, "bf16", 0), (1, 32, 512, "bf16", 0), (3, 8, 1000, "bf16", 8),
                                             (2, 4, 777, "fp32", 3), (1, 2, 4096, "bf16", 0), (1, 2, 4096, "fp32", 0),
                                             (1, 3, 2500, "fp32", 4), (1, 112, 512, "bf16", 0)])
def test_influence_drift(B, H, L, dtype, pad):
    print(f"case: influence B={B} H={H} L={L} {dtype} pad={pad}", flush=True)
    _check(B, H, L, dtype, seed=B * 1000 + H * 10 + L, pad=pad)


def test_padding_is_ignored():
    print("case: influence NaN padding", flush=True)
    _check(2, 3, 100, "bf16", seed=4, pad=4, pad_bits=0x7FC0)
    _check(2, 3, 101, "fp32", seed=5, pad=3, pad_bits=0x7FC00000)


def test_edge_masks():
    print("case: influence edge masks", flush=True)
    dev = _dev()
    t, host, _, _ = _case(1, 4, 96, "fp32", 6)
    z = torch.zeros((1, 96), dtype=torch.uint8, device=dev)
    o = torch.ones((1, 96), dtype=torch.uint8, device=dev)
    d_in, d_out = dv.dv_influence_drift(t, z, z)
    assert float(d_in.abs().max()) == 0.0 and float(d_out.abs().max()) == 0.0
    d_in, d_out = dv.dv_influence_drift(t, o, o)
    # every row hands out one unit per head: d_out is the mean row sum, d_in sums to the row count
    np.testing.assert_allclose(d_out.cpu().numpy(), 1.0, rtol=1e-5)
    np.testing.assert_allclose(float(d_in.sum()), 96.0, rtol=1e-5)


def test_cover_seed_chain():
    """COVER's seed selection end to end: d_in, d_out from attention, u from the verifier, then the score and top-k."""
    print("case: influence -> seed score -> top-k", flush=True)
    dev = _dev()
    B, H, L, k = 2, 16, 256, 32
    t, host, qm, nc = _case(B, H, L, "bf16", 8)
    rng = np.random.default_rng(9)
    u = rng.uniform(0, 10, (B, L)).astype(np.float32)
    committed = (rng.random((B, L)) < 0.5).astype(np.uint8)
    d_in, d_out = dv.dv_influence_drift(t, torch.from_numpy(qm).to(dev), torch.from_numpy(nc).to(dev))
    score = dv.dv_seed_score(torch.from_numpy(u.ravel()).to(dev), d_in.view(-1), d_out.view(-1),
                             torch.from_numpy(committed.ravel()).to(dev))
    idx, _, cnt, _ = dv.dv_select_topk(score.view(B, L), k, eligible=torch.from_numpy(committed).to(dev))
    r_in, r_out = OA.influence_drift(_widen(host, "bf16"), qm, nc)
    ref_score = OS.seed_score(u.ravel(), r_in.ravel(), r_out.ravel(), committed.ravel()).reshape(B, L)
    got = score.cpu().numpy().reshape(B, L)
    fin = np.isfinite(ref_score)
    np.testing.assert_allclose(got[fin], ref_score[fin], rtol=RTOL, atol=ATOL)
    ri, _, rc = OS.select_topk(ref_score, k, eligible=committed)
    for b in range(B):
        srt = np.sort(ref_score[b][fin[b]])[::-1]
        if srt.size > k and srt[k - 1] - srt[k] > 1e-5:
            assert set(idx.cpu().numpy()[b].tolist()) == set(ri[b].tolist())


def test_bench_shape_784_maps():
    """The launch `bench.py --influence 784` times: 784 maps (e.g. 28 layers x 28 heads) of 512 x 512 bf16
    softmax rows drawn on the device, 40% of the queries masked, 20% of the columns new."""
    print("case: influence 784 x 512 x 512 bf16 (benchmark shape)", flush=True)
    dev = _dev()
    maps, L = 784, 512
    g = torch.Generator(device=dev)
    g.manual_seed(2024)
    probs = torch.empty((1, maps, L, L), dtype=torch.bfloat16, device=dev)
    for h in range(maps):
        x = torch.randn((L, L), generator=g, device=dev, dtype=torch.float32) * 3.0
        probs[0, h].copy_(torch.softmax(x, dim=-1).to(torch.bfloat16))
    qm = (torch.rand((1, L), generator=g, device=dev) < 0.4).to(torch.uint8)
    nc = (torch.rand((1, L), generator=g, device=dev) < 0.2).to(torch.uint8)
    d_in, d_out = dv.dv_influence_drift(probs, qm, nc)
    # the prepared call bench.py times gives the same bits, call after call
    ws = torch.empty(dv.dv_influence_drift_workspace_bytes(probs) + 256, dtype=torch.uint8, device=dev)
    p_in, p_out = torch.empty_like(d_in), torch.empty_like(d_out)
    call = dv.prepare_influence_drift(probs, qm, nc, p_in, p_out, ws)
    for _ in range(3):
        p_in.fill_(-1.0)
        call()
        torch.cuda.synchronize()
        assert torch.equal(p_in, d_in) and torch.equal(p_out, d_out)
    torch.cuda.synchronize()
    host = probs.view(torch.int16).cpu().numpy().view(np.uint16)
    r_in, r_out = OA.influence_drift(_widen(host, "bf16"), qm.cpu().numpy(), nc.cpu().numpy())
    del host
    np.testing.assert_allclose(d_in.cpu().numpy(), r_in, rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(d_out.cpu().numpy(), r_out, rtol=RTOL, atol=ATOL)
    del probs
    torch.cuda.empty_cache()
