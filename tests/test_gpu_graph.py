"""A decode step captured once in a HIP graph and replayed (lca_ragged_step_graph: the lengths live on the
device, the attention launch advances them), against the eager one-call step on a twin cache: top-k lists,
outputs, LSE and cache bytes bit for bit after every replay, with eager work and synchronisations between
the replays; then a replay past the capacity it was captured for leaves the cache and the outputs alone
(CSA paragraph, Figures 3 and 4 of "DeepSeek-V4: a million-token context that agents can actually use":
the same computation as the step, position by position)."""
import numpy as np
import pytest

from long_context_attention_18_amd import configs

pytestmark = pytest.mark.gpu

try:
    from gpu_harness import LayerRun, to_dev, from_dev
except ImportError:  # run from the repository root
    from tests.gpu_harness import LayerRun, to_dev, from_dev


def _ragged_fill(run, total, chunk=8192):
    lens = np.zeros(run.B, np.int64)
    bias = run.bias_dev
    for pos in range(0, total, chunk):
        T = min(chunk, total - pos)
        parts = [run.tokens(b, pos, T) for b in range(run.B)]
        tok = {k: to_dev(np.stack([p[k] for p in parts])) for k in parts[0]}
        run.dev.ragged_ingest(lens, np.full(run.B, T, np.int32), tok["kv"], tok.get("gate"), bias.get("bias"),
                              tok.get("ik"), tok.get("ig"), bias.get("idx_bias"))
        lens += T
    run.len = total


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_graph_replay_matches_the_step(kind):
    import torch
    import long_context_attention_18_amd as lca
    if kind == "csa":
        layer, B, ctx = configs.Layer("csa", 4, n_heads=64, window=128, idx_heads=8, topk=256), 3, 9001
    else:
        layer, B, ctx = configs.Layer("hca", 128, n_heads=64, window=128), 2, 70001
    steps = 6
    cap = ctx + steps
    a = LayerRun(layer, B=B, max_ctx=cap + 8, ring=128)  # graph replays (lengths on the device)
    b = LayerRun(layer, B=B, max_ctx=cap + 8, ring=128)  # the eager one-call step
    _ragged_fill(a, ctx)
    b.fill(ctx)
    H, csa = layer.n_heads, layer.csa
    # the graph's fixed buffers: this step's tokens and queries are copied in before each replay
    parts = [a.tokens(i, ctx, 1) for i in range(B)]
    tok = {k: to_dev(np.stack([p[k] for p in parts])) for k in parts[0]}
    qd = {k: to_dev(v) for k, v in a.queries([ctx]).items()}
    out = torch.empty((B, 1, H, 128), dtype=torch.int16, device="cuda")
    lse = torch.empty((B, 1, H), dtype=torch.float32, device="cuda")
    topk = torch.full((B, 1, layer.topk), -7, dtype=torch.int32, device="cuda") if csa else None
    len_dev = torch.full((B,), ctx, dtype=torch.int64, device="cuda")
    T_dev = torch.ones((B,), dtype=torch.int32, device="cuda")
    bias = a.bias_dev
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        lca.lca_ragged_step_graph(a.dev.cache, 1, cap, len_dev, T_dev, tok["kv"], tok["gate"], tok.get("ik"),
                                  tok.get("ig"), bias["bias"], bias.get("idx_bias"), qd.get("qI") if csa else None,
                                  qd.get("w") if csa else None, qd["q"], topk, out, lse, a.dev.ws, a.dev.ws_bytes,
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert int(len_dev.cpu()[0]) == ctx  # capturing runs nothing
    for i in range(steps):
        t = ctx + i
        parts = [a.tokens(s, t, 1) for s in range(B)]
        step_tok = {k: to_dev(np.stack([p[k] for p in parts])) for k in parts[0]}
        step_q = {k: to_dev(v) for k, v in a.queries([t]).items()}
        for k in tok:
            tok[k].copy_(step_tok[k])
        for k in qd:
            qd[k].copy_(step_q[k])
        g.replay()
        torch.cuda.synchronize()
        ga = (from_dev(topk) if csa else None, from_dev(out, np.uint16), from_dev(lse))
        assert (len_dev.cpu().numpy() == t + 1).all()
        # the eager step on the twin, same inputs
        out_b = torch.empty_like(out)
        lse_b = torch.empty_like(lse)
        if csa:
            topk_b = torch.full_like(topk, -7)
            b.dev.step(step_tok["kv"], step_tok["gate"], step_tok["ik"], step_tok["ig"], bias["bias"],
                       bias["idx_bias"], step_q["qI"], step_q["w"], step_q["q"], out_b, lse_b, topk_b)
        else:
            b.dev.hca_step(step_tok["kv"], step_tok["gate"], bias["bias"], step_q["q"], out_b, lse_b)
        b.len += 1
        torch.cuda.synchronize()
        if csa:
            assert np.array_equal(ga[0], from_dev(topk_b)), i
        assert np.array_equal(ga[1], from_dev(out_b, np.uint16)), i
        assert np.array_equal(ga[2].view(np.uint32), from_dev(lse_b).view(np.uint32)), i
    va, vb = a.dev.views(), b.dev.views()
    for k in va:
        assert np.array_equal(va[k].cpu().numpy(), vb[k].cpu().numpy()), k
    # at capacity: another replay takes no step (lengths, cache bytes and outputs unchanged)
    out.fill_(-12345)
    before = {k: v.clone() for k, v in a.dev.views().items()}
    g.replay()
    torch.cuda.synchronize()
    assert (len_dev.cpu().numpy() == cap).all()
    assert (out.cpu().numpy() == -12345).all()
    for k, v in a.dev.views().items():
        assert torch.equal(v, before[k]), k
