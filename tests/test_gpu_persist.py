"""GPU parity of compressed-KV persistence (the KV-cache section of velog.io "DeepSeek V4 논문 정리":
compressed KV stored on disk for requests that share a prefix): a restored sequence holds exactly
the state of one that ingested the same tokens, and queries after a restore match the oracle run
over those tokens. Snapshots travel through a file on the way."""
import numpy as np
import pytest

from long_context_attention_18_amd import configs

pytestmark = pytest.mark.gpu

try:
    from gpu_harness import LayerRun, check_queries, compare_cache, from_dev
except ImportError:  # run from the repository root
    from tests.gpu_harness import LayerRun, check_queries, compare_cache, from_dev


def _decode_both(a, b, seq_a, n_steps, oc_b):
    """n decode steps on runs a and b (same tokens and queries for a's sequence seq_a and b's sequence 0):
    identical outputs bit for bit, and b's within the bar against the oracle."""
    for _ in range(n_steps):
        a.ingest(1)
        b.ingest(1)
        qa, ta, oa, la = a.run_queries(1)
        qb, tb, ob, lb = b.run_queries(1)
        assert np.array_equal(qa["q"][seq_a], qb["q"][0])
        if ta is not None:
            assert np.array_equal(ta[seq_a], tb[0])
        assert np.array_equal(oa[seq_a], ob[0])
        assert np.array_equal(la[seq_a].view(np.uint32), lb[0].view(np.uint32))
        check_queries(b, oc_b, qb, tb, ob, lb, [b.len - 1])


@pytest.mark.parametrize("kind", ["csa", "hca", "swa"])
def test_snapshot_restore_roundtrip_bit_exact(kind, tmp_path):
    """Sequence 1 of a B=2 cache (live tail) -> snapshot -> file -> a B=1 cache with a larger ring: the
    state and the next decode steps are those of the source, bit for bit, and match the oracle."""
    import long_context_attention_18_amd as lca
    layer = {"csa": configs.Layer("csa", 4, n_heads=32, window=128, idx_heads=4, topk=64),
             "hca": configs.Layer("hca", 128, n_heads=32, window=128),
             "swa": configs.Layer("swa", 1, n_heads=32, window=128)}[kind]
    a = LayerRun(layer, B=2, max_ctx=3000, ring=128, layer_id=3)
    for T in (1000, 7, 2):
        a.ingest(T)
    snap, info = a.dev.snapshot(1)
    assert info.len == 1009 and info.n_win == 128
    path = str(tmp_path / f"{kind}.lcas")
    lca.save_snapshot(path, snap)
    snap2, info2 = lca.load_snapshot(path)
    assert bytes(info2) == bytes(info)
    b = LayerRun(layer, B=1, max_ctx=3000, ring=200, layer_id=3, seq_ids=[1])
    b.dev.restore(snap2, info2, seq=-1)
    b.len = a.len
    assert b.dev.len == 1009
    oc_b = [b.oracle_caches(0, 1012)]
    compare_cache(b, oc_b, window_positions=128)
    _decode_both(a, b, 1, 3, oc_b)
    compare_cache(b, oc_b, window_positions=131)
    # the source's snapshot bytes equal a fresh snapshot of the restored copy, taken at the same length
    c = LayerRun(layer, B=1, max_ctx=3000, ring=128, layer_id=3, seq_ids=[1])
    c.dev.restore(snap2, info2, seq=0)
    s3, i3 = c.dev.snapshot(0)
    assert bytes(i3) == bytes(info)
    assert np.array_equal(from_dev(s3), from_dev(snap))


@pytest.mark.parametrize("kind,P", [("csa", 1001), ("hca", 1001), ("swa", 300)])
def test_shared_prefix_restored_into_every_sequence(kind, P, tmp_path):
    """A P-token prefix is compressed once (B=1), stored, and restored into all 3 sequences of another
    cache, which then continue with their own tokens (37 at once, then 3 decode steps; the HCA prefix
    ends inside a block that the suffix completes from the restored tail). Against the oracle over
    prefix + own tokens."""
    import long_context_attention_18_amd as lca
    layer = {"csa": configs.Layer("csa", 4, n_heads=16, window=128, idx_heads=8, topk=128),
             "hca": configs.Layer("hca", 128, n_heads=16, window=128),
             "swa": configs.Layer("swa", 1, n_heads=16, window=128)}[kind]
    pre = LayerRun(layer, B=1, max_ctx=P, ring=128, layer_id=4, seq_ids=[9])
    pre.ingest(P)
    snap, info = pre.dev.snapshot(0)
    path = str(tmp_path / "prefix.lcas")
    lca.save_snapshot(path, snap)
    del snap
    snap, info = lca.load_snapshot(path)
    streams = None

    def tokens(b, pos0, n):
        parts = []
        if pos0 < P:
            parts.append(pre.streams[0].tokens(pos0, min(n, P - pos0)))
        if pos0 + n > P:
            s0 = max(pos0, P)
            parts.append(streams[b].tokens(s0, pos0 + n - s0))
        return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}

    run = LayerRun(layer, B=3, max_ctx=P + 64, ring=128, layer_id=4, token_fn=tokens)
    streams = run.streams
    run.dev.restore(snap, info, seq=-1)
    run.len = P
    oc = [run.oracle_caches(b, P + 40) for b in range(3)]
    compare_cache(run, oc)
    run.ingest(37)
    qin, topk, out, lse = run.run_queries(1)
    check_queries(run, oc, qin, topk, out, lse, [run.len - 1])
    for _ in range(3):
        run.ingest(1)
        qin, topk, out, lse = run.run_queries(1)
        check_queries(run, oc, qin, topk, out, lse, [run.len - 1])
    compare_cache(run, oc)
    # the three sequences now differ (their own suffixes), but share the restored prefix state
    v = run.dev.views()
    if kind != "swa":
        nb = P // layer.m
        for b in (1, 2):
            assert np.array_equal(from_dev(v["blk_codes"][b, :nb]), from_dev(v["blk_codes"][0, :nb]))
    assert not np.array_equal(out[0], out[1])


def test_restore_one_sequence_of_a_batch():
    """Sequence 1 of a B=2 CSA cache replaced by another cache's sequence at the same length; sequence 0
    keeps its own state. Both against the oracle over their tokens."""
    layer = configs.Layer("csa", 4, n_heads=16, window=128, idx_heads=4, topk=64)
    src = LayerRun(layer, B=1, max_ctx=1200, ring=128, layer_id=5, seq_ids=[7])
    src.ingest(1001)
    snap, info = src.dev.snapshot(0)
    run = LayerRun(layer, B=2, max_ctx=1200, ring=128, layer_id=5)
    run.ingest(1001)     # sequence 1 first holds the tokens of seeded sequence 1 ...
    run.dev.restore(snap, info, seq=1)   # ... then seeded sequence 7's state and, from here on, its inputs
    run.streams[1] = src.streams[0]
    run.seq_ids[1] = 7
    oc = [run.oracle_caches(b, 1004) for b in range(2)]
    compare_cache(run, oc)
    for _ in range(3):
        run.ingest(1)
        qin, topk, out, lse = run.run_queries(1)
        check_queries(run, oc, qin, topk, out, lse, [run.len - 1])
