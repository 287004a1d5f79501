"""The one-launch indexer path of the CSA decode calls (scores, each score workgroup's own candidates, and
the top-k selection by the last workgroup of each query, all in one launch; CSA paragraph of "DeepSeek-V4:
a million-token context that agents can actually use": top-k compressed blocks per query by the lightning
indexer's scores) on its exact side paths:
  * a crowded chunk: one 2048-block chunk holds most of every query's winners, more than its own
    candidates cover, so the selecting workgroup takes the keys above the lowest candidate floor from the
    query's key row in memory -- through lca_csa_step and lca_csa_attend, against the oracle (and, through
    the harness, against the separate score and selection calls);
  * separate score calls without their selection before it (histogram counts left behind, which the
    one-launch path does not read) -- still the oracle's lists, at 2750 and 10250 blocks.
"""
import numpy as np
import pytest

from long_context_attention_18_amd import configs, synth

pytestmark = pytest.mark.gpu

try:
    from gpu_harness import LayerRun, check_queries, compare_cache, to_dev
except ImportError:  # run from the repository root
    from tests.gpu_harness import LayerRun, check_queries, compare_cache, to_dev


def _crowd(lo_blk, hi_blk):
    def transform(tok, pos0):
        f = synth.bf16_to_f32(tok["ik"]).copy()
        blk = (pos0 + np.arange(f.shape[0])) // 4
        f[(blk >= lo_blk) & (blk < hi_blk)] *= np.float32(8.0)
        out = dict(tok)
        out["ik"] = synth.bf16_bits(f)
        return out
    return transform


def _positive_weights(qin):
    out = dict(qin)
    out["w"] = np.abs(qin["w"])
    return out


def test_crowded_chunk_is_selected_from_every_key():
    """Blocks 4096-6143 (score chunk 2 of 5) get their indexer keys scaled 8x and every weight is positive:
    nearly all of each query's top-256 sit in that chunk, whose own candidates stop well above the bound, so
    the selecting workgroup takes the whole key row. B = 2, 40000 tokens, decode steps through lca_csa_step
    and lca_csa_attend: lists and scores equal the oracle's."""
    layer = configs.Layer("csa", 4, n_heads=16, window=128, idx_heads=8, topk=256)
    run = LayerRun(layer, B=2, max_ctx=40016, ring=128, sigma=1.0, transform=_crowd(4096, 6144),
                   qtransform=_positive_weights)
    run.fill(40000)
    oc = [run.oracle_caches(i, 40008) for i in range(run.B)]
    for i in range(4):
        if i % 2 == 0:
            qin, tk, out, lse = run.step(1)
        else:
            run.ingest(1)
            qin, tk, out, lse = run.run_queries(1, fused=True)
        crowded = ((tk >= 4096) & (tk < 6144)).sum(axis=-1)
        assert (crowded > 200).all(), crowded
        w = check_queries(run, oc, qin, tk, out, lse, [run.len - 1])
        assert w["scores_checked"] > 0
    compare_cache(run, oc)


@pytest.mark.parametrize("ctx", [11000, 41000])
def test_threshold_after_a_score_call_without_selection(ctx):
    """Two lca_csa_index_score calls leave their counts in the histograms; the one-launch calls after them
    (lca_csa_attend, then lca_csa_step) select from their own records and are unaffected: lists equal the
    oracle's."""
    layer = configs.Layer("csa", 4, n_heads=16, window=128, idx_heads=8, topk=256)
    run = LayerRun(layer, B=2, max_ctx=ctx + 8, ring=128)
    run.fill(ctx)
    oc = [run.oracle_caches(i, ctx + 4) for i in range(run.B)]
    for _ in range(2):
        run.ingest(1)
        qin = run.queries([run.len - 1])
        for _ in range(2):
            run.dev.index_score(to_dev(qin["qI"]), to_dev(qin["w"]))
        qa, tk, out, lse = run.run_queries(1, fused=True)
        check_queries(run, oc, qa, tk, out, lse, [run.len - 1])
    for _ in range(2):
        qa, tk, out, lse = run.step(1)
        check_queries(run, oc, qa, tk, out, lse, [run.len - 1])


# one indexer key input for every token: a quarter of FP4 grid values (exact in bf16; the pooled key is
# the same vector up to the last bits of fp64, which the FP4 codes and their power-of-two scale ignore:
# the largest magnitude 1.5 is no power of two and every element sits on the grid)
_GRID = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 1.0], np.float32)
_IK = (0.25 * _GRID[np.arange(64) % 8] * np.where(np.arange(64) % 3 == 0, -1.0, 1.0)).astype(np.float32)


def _same_key(tok, pos0):
    """Every token's indexer key input is _IK: every pooled indexer key, hence every score, is equal."""
    out = dict(tok)
    out["ik"] = synth.bf16_bits(np.broadcast_to(_IK, tok["ik"].shape).copy())
    return out


@pytest.mark.parametrize("ctx", [20001, 41001])
def test_all_scores_equal_select_the_first_blocks(ctx):
    """Every block gets the same indexer key, so every score ties: the top-k are the k lowest blocks. No
    record can hold any key (each chunk's 2048 equal keys overflow it in one sub-bin), so the selecting
    workgroup takes the key row: 5000 visible blocks (they fit its LDS) or 10250 (more than fit: straight
    from memory). Lists, scores and outputs against the oracle, through lca_csa_step and lca_csa_attend."""
    layer = configs.Layer("csa", 4, n_heads=16, window=128, idx_heads=8, topk=256)
    run = LayerRun(layer, B=2, max_ctx=ctx + 8, ring=128, transform=_same_key)
    run.fill(ctx)
    oc = [run.oracle_caches(i, ctx + 4) for i in range(run.B)]
    for i in range(3):
        if i % 2 == 0:
            qin, tk, out, lse = run.step(1)
        else:
            run.ingest(1)
            qin, tk, out, lse = run.run_queries(1, fused=True)
        scores = run.last_scores
        if scores is not None:
            s = scores[:, 0, : run.len // 4]
            assert (s == s[:, :1]).all(), "the transform should make every score equal"
        assert (tk == np.arange(layer.topk)).all(), tk[:, 0, :8]
        check_queries(run, oc, qin, tk, out, lse, [run.len - 1])
