"""The whole path under HIP graph capture: dv_verify_rows (with its noise table),
dv_decide, dv_seed_score, dv_select_topk, dv_seed_select, dv_decide_seed_select and
dv_seed_select_decide allocate nothing and clear nothing
with memset, so a captured step replays to the eager results, replay after
replay, with other work and synchronisations in between."""

import numpy as np
import pytest
import torch

import token_verification_row_amd as dv
import workloads as W

pytestmark = pytest.mark.gpu


def _step(a, b, w, out, ws, d_in, d_out, bufs):
    got = dv.dv_verify_rows(a, b, temperature=w.temperature, seed=w.seed, pos_period=w.pos_period, out=out,
                            workspace=ws)
    d, o, pre, best = dv.dv_decide("COUPLED_ACCEPT", got, mask_token=-1, group_len=w.group_len, want_prefix=True,
                                   want_best=True)
    score = dv.dv_seed_score(got["entropy"], d_in, d_out)
    idx, val, cnt, _ = dv.dv_select_topk(score.view(-1, w.group_len), 8)
    # the same seed score and selection in one launch
    score2, idx2, val2, cnt2, _ = dv.dv_seed_select(got["entropy"].view(-1, w.group_len), d_in, d_out, 8)
    # the decisions and the seed selection in one launch
    (d3, o3, pre3, best3), (score3, idx3, _, cnt3, _) = dv.dv_decide_seed_select(
        dict(rule="COUPLED_ACCEPT", stats=got, mask_token=-1, group_len=w.group_len, want_prefix=True, want_best=True),
        dict(u=got["entropy"].view(-1, w.group_len), d_in=d_in.view(-1, w.group_len),
             d_out=d_out.view(-1, w.group_len), k=8))
    # COVER's seed step: the selection, then the decisions over its seeds, in one launch
    (_, _, _, _, mask4), (d4, o4) = dv.dv_seed_select_decide(
        dict(u=got["entropy"].view(-1, w.group_len), d_in=d_in.view(-1, w.group_len),
             d_out=d_out.view(-1, w.group_len), k=8),
        dict(rule="COVER", stats=got, conf_thr=0.9, mask_token=-1))
    for k, v in (("d", d), ("o", o), ("pre", pre), ("best", best), ("idx", idx), ("val", val), ("cnt", cnt),
                 ("score2", score2), ("idx2", idx2), ("val2", val2), ("cnt2", cnt2), ("d3", d3), ("o3", o3),
                 ("pre3", pre3), ("best3", best3), ("score3", score3), ("idx3", idx3), ("cnt3", cnt3),
                 ("mask4", mask4), ("d4", d4), ("o4", o4)):
        bufs[k] = v
    return bufs


def test_path_replays_in_a_graph():
    print("case: graph capture of the path", flush=True)
    dev = torch.device("cuda:0")
    w = W.workload(4)
    rows, V = 256, 8192                      # 8 candidates x 32 positions, shared noise per position
    rng = np.random.default_rng(0)
    a_np = (rng.standard_normal((rows, V)) * 2).astype(np.float32)
    b_np = a_np + (rng.standard_normal((rows, V)) * 0.5).astype(np.float32)
    a = torch.from_numpy(W.round_bf16_bits(a_np).view(np.int16)).to(dev).view(torch.bfloat16)
    b = torch.from_numpy(W.round_bf16_bits(b_np).view(np.int16)).to(dev).view(torch.bfloat16)
    d_in = torch.rand(rows, device=dev)
    d_out = torch.rand(rows, device=dev)
    need = dv.dv_verify_workspace_bytes(a, b, temperature=w.temperature, seed=w.seed, pos_period=w.pos_period)
    assert need > 0                          # the noise table is part of the captured work
    ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    out = {k: torch.empty(rows, dtype=torch.float32 if k in ("lse_v", "lse_d", "kl", "entropy", "conf") else torch.int32,
                          device=dev) for k in dv.CORE_FIELDS}
    eager = {k: v.clone() for k, v in _step(a, b, w, out, ws, d_in, d_out, {}).items()}
    for x, y in (("d", "d3"), ("o", "o3"), ("pre", "pre3"), ("best", "best3"), ("score2", "score3"), ("idx2", "idx3"),
                 ("cnt2", "cnt3")):
        assert torch.equal(eager[x].view(-1), eager[y].view(-1)), (x, y)
    eager_stats = {k: v.clone() for k, v in out.items()}
    torch.cuda.synchronize()

    # capture on a side stream (torch's graph capture); outputs of the graph live in its private pool
    for v in out.values():
        v.zero_()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(a, b, w, out, ws, d_in, d_out, {})     # warm the allocator on this stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    bufs = {}
    with torch.cuda.graph(g):
        _step(a, b, w, out, ws, d_in, d_out, bufs)
    for replay in range(4):
        for v in out.values():
            v.fill_(-7)                              # stale values must be overwritten
        junk = torch.randn(1 << 20, device=dev).sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for k in eager_stats:
            assert torch.equal(out[k], eager_stats[k]), (replay, k)
        for k in eager:
            assert torch.equal(bufs[k], eager[k]), (replay, k)
        del junk
