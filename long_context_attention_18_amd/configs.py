"""The synthetic workloads and the closed forms of their bytes.

Every layer shares the entry format the storage paragraph of the pages fixes
in kind ("DeepSeek-V4: a million-token context that agents can actually use":
FP8 KV entries, BF16 RoPE dims, FP4 indexer): one 196-byte entry (64 FP8
codes + one fp32 scale + 64 BF16 RoPE values) per compressed block or
window token, and a 34-byte indexer key (64 FP4 codes + two E8M0 scale
bytes) per CSA block.
"""
from __future__ import annotations

from dataclasses import dataclass, field

ENTRY_BYTES = 64 + 4 + 128      # FP8 nope + fp32 scale + BF16 rope
IDX_KEY_BYTES = 32 + 2          # 64 x FP4 + 2 x E8M0
GQA8_BF16_BYTES_PER_TOKEN = 2 * 8 * 128 * 2   # K and V, 8 heads, dim 128, 2 bytes


@dataclass(frozen=True)
class Layer:
    kind: str            # "csa", "hca" or "swa" (window only: no compressed stream)
    m: int               # tokens per compressed entry (4 / 128; 1 and unused for "swa")
    n_heads: int = 64    # query heads, dim 128
    window: int = 128
    idx_heads: int = 0   # CSA indexer heads (dim 64)
    topk: int = 0        # CSA top-k

    @property
    def csa(self) -> bool:
        return self.kind == "csa"

    @property
    def swa(self) -> bool:
        return self.kind == "swa"

    def blocks(self, context: int) -> int:
        """Compressed entries one sequence holds at `context` tokens (none for a window-only layer)."""
        return 0 if self.swa else context // self.m


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    layers: tuple
    batch: int
    context: int          # tokens already cached before the first query
    hidden: int
    decode_steps: int = 1
    prefill_chunk: int = 0
    sigma: float = 0.0    # std of directly drawn per-token inputs
    note: str = ""
    shared_streams: bool = False  # layers of one kind read one token stream (deep stacks: cheaper to fill)

    def layer(self, i: int) -> Layer:
        return self.layers[i]


def _csa(H, HI, k, W=128):
    return Layer("csa", 4, n_heads=H, window=W, idx_heads=HI, topk=k)


def _hca(H, W=128):
    return Layer("hca", 128, n_heads=H, window=W)


def _swa(H, W=128):
    return Layer("swa", 1, n_heads=H, window=W)


def v4pro_schedule(n_layers: int = 61, mtp: bool = True) -> tuple:
    """Layer kinds of V4-Pro's stack as the layer interleave paragraph of the pages gives it: layers 0-1
    HCA, layers 2..n_layers-1 alternating CSA and HCA (CSA first), then the final MTP block, which runs
    only the sliding window."""
    kinds = ["hca", "hca"] + ["csa" if (i - 2) % 2 == 0 else "hca" for i in range(2, n_layers)]
    return tuple(kinds + (["swa"] if mtp else []))


def _stack(kinds, H=64, HI=8, k=1024):
    return tuple(_csa(H, HI, k) if x == "csa" else (_hca(H) if x == "hca" else _swa(H)) for x in kinds)


WORKLOADS = {
    0: Workload(0, "csa_decode_small", (_csa(8, 4, 64),), batch=1, context=4096, hidden=1024, decode_steps=16,
                sigma=0.02 * 1024 ** 0.5,
                note="CSA, B=1, 4096-token context, 16 consecutive decode queries, H=8, H_I=4, k=64"),
    1: Workload(1, "hca_decode_64k", (_hca(64),), batch=8, context=65536, hidden=4096, decode_steps=1,
                sigma=0.02 * 4096 ** 0.5, note="HCA, B=8, 65536-token context, H=64"),
    2: Workload(2, "csa_decode_1m", (_csa(64, 8, 1024),), batch=4, context=1 << 20, hidden=4096,
                decode_steps=1, sigma=0.02 * 4096 ** 0.5,
                note="CSA, B=4, 1,048,576-token context, H=64, H_I=8, k=1024"),
    3: Workload(3, "csa_prefill_128k", (_csa(64, 8, 512),), batch=1, context=0, hidden=4096, prefill_chunk=8192,
                decode_steps=0, sigma=1.0, note="CSA chunked prefill of 131072 tokens, chunk 8192, k=512"),
    4: Workload(4, "stack8_decode_256k", _stack(v4pro_schedule(8, mtp=False)),
                batch=16, context=262144, hidden=4096, decode_steps=1, sigma=0.02 * 4096 ** 0.5,
                note="8 layers HCA,HCA,CSA,HCA,CSA,HCA,CSA,HCA; B=16, 262144-token context"),
    5: Workload(5, "v4pro61_mtp_decode_1m", _stack(v4pro_schedule(61, mtp=True)),
                batch=4, context=1 << 20, hidden=4096, decode_steps=1, sigma=0.02 * 4096 ** 0.5,
                note="V4-Pro's 61-layer interleave (HCA,HCA, then CSA/HCA alternating: 30 CSA + 31 HCA) plus "
                     "the window-only MTP block; B=4, 1,048,576-token context; layers of one kind share one "
                     "token stream (own pooling biases and queries per layer)", shared_streams=True),
}

PREFILL_TOKENS = {3: 131072}


def stream_layer_id(wl: Workload, li: int) -> int:
    """Layer id that seeds layer li's token stream: its own, or with shared streams that of the first
    layer reading the same kind of stream (the CSA stream carries the indexer inputs; HCA and window-only
    layers read the same kv stream)."""
    if not wl.shared_streams:
        return li
    csa = wl.layers[li].csa
    return next(i for i, l in enumerate(wl.layers) if l.csa == csa)


def kv_bytes_per_seq(layer: Layer, context: int) -> int:
    """Entries (compressed + window) + indexer keys one sequence keeps at `context` tokens.

    The uncompressed tail (context mod m tokens) and the sequence length are
    bookkeeping outside this count, as is any ring slack beyond the window.
    """
    n = layer.blocks(context)
    b = n * ENTRY_BYTES + min(context, layer.window) * ENTRY_BYTES
    if layer.csa:
        b += n * IDX_KEY_BYTES
    return b


def decode_step_bytes(layer: Layer, context_after_append: int) -> int:
    """Algorithmic HBM bytes of one decode query of one sequence.

    Reads: indexer keys of every visible block (CSA), the selected (CSA) or
    all visible (HCA) entries, the window entries, the query (and qI, w);
    writes: the output. The new token's own entry/tail writes are < 1 KB and
    are included as the token's inputs (kv, gate, ik, ig BF16) plus one
    window entry.
    """
    t = context_after_append - 1
    n = layer.blocks(t + 1)
    w = min(layer.window, t + 1)
    b = 0
    if layer.csa:
        b += n * IDX_KEY_BYTES
        b += min(layer.topk, n) * ENTRY_BYTES
        b += layer.idx_heads * 64 * 2 + layer.idx_heads * 4
    else:
        b += n * ENTRY_BYTES
    b += w * ENTRY_BYTES
    b += layer.n_heads * 128 * 2 * 2     # q in, out
    # the new token: kv (+ gate, and ik/ig for CSA, where a compressor reads them) and its window entry
    b += 128 * 2 * (1 if layer.swa else 2) + (64 * 2 * 2 if layer.csa else 0) + ENTRY_BYTES
    return b
