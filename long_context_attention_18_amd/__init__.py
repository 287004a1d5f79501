"""Python binding of liblca.so (include/lca.h): hybrid compressed long-context
attention -- CSA / HCA compressed KV cache with a sliding window -- on AMD
gfx950 (MI355X).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels. Functions carry the C entry points' names and arguments; device
buffers may be passed as torch tensors (their data_ptr() is used) or as raw
integer addresses. A non-zero status raises ``LcaError``. There is no CPU
fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblca.so")

LCA_KIND_CSA = 0
LCA_KIND_HCA = 1
LCA_KIND_SWA = 2
_KINDS = {"csa": LCA_KIND_CSA, "hca": LCA_KIND_HCA, "swa": LCA_KIND_SWA}

_STATUS = {0: "LCA_OK", -1: "LCA_ERR_NULL", -2: "LCA_ERR_SHAPE", -3: "LCA_ERR_UNSUPPORTED", -4: "LCA_ERR_CAPACITY",
           -5: "LCA_ERR_ORDER", -6: "LCA_ERR_WORKSPACE", -7: "LCA_ERR_LAUNCH"}


class LcaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {_STATUS.get(status, status)} ({lib().lca_status_str(status).decode()})")


class lca_layer_desc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("m", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("window", ctypes.c_int32), ("idx_heads", ctypes.c_int32), ("topk", ctypes.c_int32)]


class lca_cache(ctypes.Structure):
    _fields_ = [("desc", lca_layer_desc), ("batch", ctypes.c_int32), ("ring", ctypes.c_int32),
                ("max_ctx", ctypes.c_int64), ("max_blocks", ctypes.c_int64), ("len", ctypes.c_int64),
                ("pending", ctypes.c_int64),
                ("blk_codes_dev", ctypes.c_void_p), ("blk_scale_dev", ctypes.c_void_p),
                ("blk_rope_dev", ctypes.c_void_p), ("idx_codes_dev", ctypes.c_void_p),
                ("idx_scale_dev", ctypes.c_void_p), ("win_codes_dev", ctypes.c_void_p),
                ("win_scale_dev", ctypes.c_void_p), ("win_rope_dev", ctypes.c_void_p),
                ("tail_dev", ctypes.c_void_p), ("tail_width", ctypes.c_int32), ("ragged", ctypes.c_int32),
                ("rope_inv_freq", ctypes.c_double * 32), ("rope_inv_freq_dev", ctypes.c_void_p)]


class lca_snapshot_info(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("kind", ctypes.c_int32),
                ("m", ctypes.c_int32), ("tail_width", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("len", ctypes.c_int64), ("n_blocks", ctypes.c_int64), ("n_win", ctypes.c_int64),
                ("n_tail", ctypes.c_int64), ("off", ctypes.c_uint64 * 10), ("bytes", ctypes.c_uint64)]


LCA_SNAPSHOT_HEADER = 256

_LIB = None
_VP = ctypes.c_void_p
_DP = ctypes.POINTER(lca_layer_desc)
_CP = ctypes.POINTER(lca_cache)
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_SP = ctypes.POINTER(lca_snapshot_info)

_SIGNATURES = {
    "lca_cache_bytes": (_SZ, [_DP, _I32, _I64, _I32]),
    "lca_cache_bind": (_I32, [_DP, _CP, _VP, _SZ, _I32, _I64, _I32, _VP]),
    "lca_workspace_bytes": (_SZ, [_DP, _I32, _I32, _I64]),
    "lca_workspace_init": (_I32, [_VP, _SZ, _VP]),
    "lca_workspace_scores_offset": (_SZ, [_DP, _I32, _I32, _I64]),
    "lca_csa_compress": (_I32, [_CP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP]),
    "lca_hca_compress": (_I32, [_CP, _VP, _VP, _VP, _I32, _VP]),
    "lca_swa_tail_append": (_I32, [_CP, _VP, _VP, _VP, _VP, _I32, _VP]),
    "lca_csa_indexer_topk": (_I32, [_CP, _VP, _VP, _I32, _VP, _VP, _SZ, _VP]),
    "lca_csa_index_score": (_I32, [_CP, _VP, _VP, _I32, _VP, _SZ, _VP]),
    "lca_csa_topk_select": (_I32, [_CP, _I32, _VP, _VP, _SZ, _VP]),
    "lca_csa_sparse_attn": (_I32, [_CP, _VP, _VP, _I32, _VP, _VP, _VP, _SZ, _VP]),
    "lca_hca_dense_attn": (_I32, [_CP, _VP, _I32, _VP, _VP, _VP, _SZ, _VP]),
    "lca_swa_attn": (_I32, [_CP, _VP, _I32, _VP, _VP, _VP, _SZ, _VP]),
    "lca_csa_attend": (_I32, [_CP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "lca_csa_topk_attn": (_I32, [_CP, _VP, _I32, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "lca_csa_step": (_I32, [_CP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "lca_csa_step_timed": (_I32, [_CP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ,
                                  _VP, _VP]),
    "lca_csa_step_noalloc": (_I32, [_CP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "lca_csa_step_launches": (_I32, [_CP, _I32, _VP, _SZ, ctypes.POINTER(ctypes.c_int32)]),
    "lca_hca_step": (_I32, [_CP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "lca_swa_step": (_I32, [_CP, _VP, _I32, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "lca_snapshot_layout": (_I32, [_CP, _SP]),
    "lca_cache_snapshot": (_I32, [_CP, _I32, _VP, _SZ, _SP, _VP]),
    "lca_cache_restore": (_I32, [_CP, _I32, _VP, _SZ, _SP, _VP]),
    "lca_ragged_ingest": (_I32, [_CP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "lca_ragged_step": (_I32, [_CP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                               _VP, _VP, _VP, _SZ, _VP]),
    "lca_ragged_step_graph": (_I32, [_CP, _I32, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                     _VP, _VP, _VP, _SZ, _VP]),
    "lca_ragged_snapshot": (_I32, [_CP, _I32, _I64, _VP, _SZ, _SP, _VP]),
    "lca_status_str": (ctypes.c_char_p, [_I32]),
}


def lib():
    """Load the in-tree liblca.so. Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(or python -m long_context_attention_18_amd._build)")
        # torch first: its libamdhip64 carries the soname liblca.so asks for, so both share one HIP runtime
        # (and torch's streams and events are valid in the library)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _ptr(x):
    """Device address of a torch tensor (or an int / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != 0:
        raise LcaError(fn, status)


def make_desc(kind: str, m: int, n_heads: int, window: int = 128, idx_heads: int = 0, topk: int = 0):
    """kind: "csa", "hca" or "swa" (window-only; m is then ignored)."""
    return lca_layer_desc(_KINDS[kind], m, n_heads, window, idx_heads, topk)


# ----------------------------------------------------------------- entry points
def lca_cache_bytes(desc, batch, max_ctx, ring):
    return lib().lca_cache_bytes(ctypes.byref(desc), batch, max_ctx, ring)


def lca_cache_bind(desc, cache, base, nbytes, batch, max_ctx, ring, stream=None):
    _check("lca_cache_bind", lib().lca_cache_bind(ctypes.byref(desc), ctypes.byref(cache), _ptr(base), nbytes,
                                                   batch, max_ctx, ring, _stream(stream)))


def lca_workspace_bytes(desc, batch, max_tq, max_ctx):
    return lib().lca_workspace_bytes(ctypes.byref(desc), batch, max_tq, max_ctx)


def lca_workspace_init(ws, nbytes, stream=None):
    _check("lca_workspace_init", lib().lca_workspace_init(_ptr(ws), nbytes, _stream(stream)))


def lca_workspace_scores_offset(desc, batch, query, max_ctx):
    return lib().lca_workspace_scores_offset(ctypes.byref(desc), batch, query, max_ctx)


def lca_csa_compress(cache, kv, gate, ik, ig, bias, idx_bias, T, stream=None):
    _check("lca_csa_compress", lib().lca_csa_compress(ctypes.byref(cache), _ptr(kv), _ptr(gate), _ptr(ik), _ptr(ig),
                                                       _ptr(bias), _ptr(idx_bias), T, _stream(stream)))


def lca_hca_compress(cache, kv, gate, bias, T, stream=None):
    _check("lca_hca_compress", lib().lca_hca_compress(ctypes.byref(cache), _ptr(kv), _ptr(gate), _ptr(bias), T,
                                                       _stream(stream)))


def lca_swa_tail_append(cache, kv, gate, ik, ig, T, stream=None):
    _check("lca_swa_tail_append", lib().lca_swa_tail_append(ctypes.byref(cache), _ptr(kv), _ptr(gate), _ptr(ik),
                                                             _ptr(ig), T, _stream(stream)))


def lca_csa_indexer_topk(cache, qI, w, Tq, topk, ws, ws_bytes, stream=None):
    _check("lca_csa_indexer_topk", lib().lca_csa_indexer_topk(ctypes.byref(cache), _ptr(qI), _ptr(w), Tq, _ptr(topk),
                                                               _ptr(ws), ws_bytes, _stream(stream)))


def lca_csa_index_score(cache, qI, w, Tq, ws, ws_bytes, stream=None):
    _check("lca_csa_index_score", lib().lca_csa_index_score(ctypes.byref(cache), _ptr(qI), _ptr(w), Tq, _ptr(ws),
                                                             ws_bytes, _stream(stream)))


def lca_csa_topk_select(cache, Tq, topk, ws, ws_bytes, stream=None):
    _check("lca_csa_topk_select", lib().lca_csa_topk_select(ctypes.byref(cache), Tq, _ptr(topk), _ptr(ws), ws_bytes,
                                                             _stream(stream)))


def lca_csa_sparse_attn(cache, q, topk, Tq, out, lse, ws, ws_bytes, stream=None):
    _check("lca_csa_sparse_attn", lib().lca_csa_sparse_attn(ctypes.byref(cache), _ptr(q), _ptr(topk), Tq, _ptr(out),
                                                             _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def lca_hca_dense_attn(cache, q, Tq, out, lse, ws, ws_bytes, stream=None):
    _check("lca_hca_dense_attn", lib().lca_hca_dense_attn(ctypes.byref(cache), _ptr(q), Tq, _ptr(out), _ptr(lse),
                                                           _ptr(ws), ws_bytes, _stream(stream)))


def lca_swa_attn(cache, q, Tq, out, lse, ws, ws_bytes, stream=None):
    _check("lca_swa_attn", lib().lca_swa_attn(ctypes.byref(cache), _ptr(q), Tq, _ptr(out), _ptr(lse), _ptr(ws),
                                               ws_bytes, _stream(stream)))


def lca_csa_attend(cache, qI, w, q, Tq, topk, out, lse, ws, ws_bytes, stream=None):
    _check("lca_csa_attend", lib().lca_csa_attend(ctypes.byref(cache), _ptr(qI), _ptr(w), _ptr(q), Tq, _ptr(topk),
                                                   _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def lca_csa_topk_attn(cache, q, Tq, topk, out, lse, ws, ws_bytes, stream=None):
    _check("lca_csa_topk_attn", lib().lca_csa_topk_attn(ctypes.byref(cache), _ptr(q), Tq, _ptr(topk), _ptr(out),
                                                         _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def lca_csa_step(cache, kv, gate, ik, ig, bias, idx_bias, T, qI, w, q, topk, out, lse, ws, ws_bytes, stream=None):
    _check("lca_csa_step", lib().lca_csa_step(ctypes.byref(cache), _ptr(kv), _ptr(gate), _ptr(ik), _ptr(ig),
                                               _ptr(bias), _ptr(idx_bias), T, _ptr(qI), _ptr(w), _ptr(q), _ptr(topk),
                                               _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def lca_csa_step_timed(cache, kv, gate, ik, ig, bias, idx_bias, T, qI, w, q, topk, out, lse, ws, ws_bytes, stream,
                       events):
    """events: 4 hipEvent_t handles (or None), recorded between the step's launches."""
    arr = (ctypes.c_void_p * 4)(*events)
    _check("lca_csa_step_timed", lib().lca_csa_step_timed(ctypes.byref(cache), _ptr(kv), _ptr(gate), _ptr(ik),
                                                           _ptr(ig), _ptr(bias), _ptr(idx_bias), T, _ptr(qI), _ptr(w),
                                                           _ptr(q), _ptr(topk), _ptr(out), _ptr(lse), _ptr(ws),
                                                           ws_bytes, _stream(stream), arr))


def lca_csa_step_launches(cache, T, ws, ws_bytes):
    """Kernel launches lca_csa_step makes after the compress launch: 1, 2 or 3."""
    n = ctypes.c_int32(0)
    _check("lca_csa_step_launches", lib().lca_csa_step_launches(ctypes.byref(cache), T, _ptr(ws), ws_bytes,
                                                                 ctypes.byref(n)))
    return n.value


def lca_csa_step_noalloc(cache, kv, gate, ik, ig, bias, idx_bias, T, qI, w, q, topk, out, lse, stream=None):
    _check("lca_csa_step_noalloc", lib().lca_csa_step_noalloc(
        ctypes.byref(cache), _ptr(kv), _ptr(gate), _ptr(ik), _ptr(ig), _ptr(bias), _ptr(idx_bias), T, _ptr(qI),
        _ptr(w), _ptr(q), _ptr(topk), _ptr(out), _ptr(lse), _stream(stream)))


def lca_hca_step(cache, kv, gate, bias, T, q, out, lse, ws, ws_bytes, stream=None):
    _check("lca_hca_step", lib().lca_hca_step(ctypes.byref(cache), _ptr(kv), _ptr(gate), _ptr(bias), T, _ptr(q),
                                               _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def lca_swa_step(cache, kv, T, q, out, lse, ws, ws_bytes, stream=None):
    _check("lca_swa_step", lib().lca_swa_step(ctypes.byref(cache), _ptr(kv), T, _ptr(q), _ptr(out), _ptr(lse),
                                               _ptr(ws), ws_bytes, _stream(stream)))


def lca_snapshot_layout(cache):
    info = lca_snapshot_info()
    _check("lca_snapshot_layout", lib().lca_snapshot_layout(ctypes.byref(cache), ctypes.byref(info)))
    return info


def lca_cache_snapshot(cache, seq, dst, nbytes, stream=None):
    info = lca_snapshot_info()
    _check("lca_cache_snapshot", lib().lca_cache_snapshot(ctypes.byref(cache), seq, _ptr(dst), nbytes,
                                                           ctypes.byref(info), _stream(stream)))
    return info


def lca_cache_restore(cache, seq, src, nbytes, info, stream=None):
    _check("lca_cache_restore", lib().lca_cache_restore(ctypes.byref(cache), seq, _ptr(src), nbytes,
                                                         ctypes.byref(info), _stream(stream)))


def lca_ragged_ingest(cache, T_max, len_host, T_host, len_dev, T_dev, kv, gate, ik, ig, bias, idx_bias,
                      stream=None):
    """len_host / T_host: numpy int64 / int32 arrays [B] (the same values as len_dev / T_dev)."""
    _check("lca_ragged_ingest", lib().lca_ragged_ingest(
        ctypes.byref(cache), T_max, len_host.ctypes.data, T_host.ctypes.data, _ptr(len_dev), _ptr(T_dev), _ptr(kv),
        _ptr(gate), _ptr(ik), _ptr(ig), _ptr(bias), _ptr(idx_bias), _stream(stream)))


def lca_ragged_step(cache, T_max, len_host, T_host, len_dev, T_dev, kv, gate, ik, ig, bias, idx_bias, qI, w, q, topk,
                    out, lse, ws, ws_bytes, stream=None):
    _check("lca_ragged_step", lib().lca_ragged_step(
        ctypes.byref(cache), T_max, len_host.ctypes.data, T_host.ctypes.data, _ptr(len_dev), _ptr(T_dev), _ptr(kv),
        _ptr(gate), _ptr(ik), _ptr(ig), _ptr(bias), _ptr(idx_bias), _ptr(qI), _ptr(w), _ptr(q), _ptr(topk),
        _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def lca_ragged_step_graph(cache, T_max, cap_len, len_dev, T_dev, kv, gate, ik, ig, bias, idx_bias, qI, w, q, topk, out,
                          lse, ws, ws_bytes, stream=None):
    _check("lca_ragged_step_graph", lib().lca_ragged_step_graph(
        ctypes.byref(cache), T_max, cap_len, _ptr(len_dev), _ptr(T_dev), _ptr(kv), _ptr(gate), _ptr(ik), _ptr(ig),
        _ptr(bias), _ptr(idx_bias), _ptr(qI), _ptr(w), _ptr(q), _ptr(topk), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
        _stream(stream)))


def lca_ragged_snapshot(cache, seq, length, dst, nbytes, stream=None):
    info = lca_snapshot_info()
    _check("lca_ragged_snapshot", lib().lca_ragged_snapshot(ctypes.byref(cache), seq, length, _ptr(dst), nbytes,
                                                             ctypes.byref(info), _stream(stream)))
    return info


def lca_status_str(status):
    return lib().lca_status_str(status).decode()


# ----------------------------------------------------------------- device-memory plumbing
class DeviceLayer:
    """One layer's cache and workspace in torch-allocated device memory.

    Owns the buffers (torch uint8 tensors) and the bound lca_cache struct;
    the methods forward to the entry points above with this layer's cache.
    """

    def __init__(self, desc, batch, max_ctx, ring, max_tq=1, device="cuda", stream=None):
        import torch
        self.desc = desc
        self.batch, self.max_ctx, self.ring, self.max_tq = batch, max_ctx, ring, max_tq
        nbytes = lca_cache_bytes(desc, batch, max_ctx, ring)
        if nbytes == 0:
            raise LcaError("lca_cache_bytes", -2)
        self.cache_bytes = nbytes
        self.mem = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = (self.mem.data_ptr() + 255) // 256 * 256
        self.cache = lca_cache()
        lca_cache_bind(desc, self.cache, base, nbytes, batch, max_ctx, ring, stream)
        self.ws_bytes = lca_workspace_bytes(desc, batch, max_tq, max_ctx)
        self.ws_mem = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=device)
        self.ws = (self.ws_mem.data_ptr() + 255) // 256 * 256
        lca_workspace_init(self.ws, self.ws_bytes, stream)

    def replica(self, stream=None):
        """A second cache with this one's contents in new device memory (bound, then a byte copy of the cache
        memory, len and pending copied): the same state at other addresses. It shares this layer's
        workspace, so calls on the two must not overlap in time."""
        import copy
        import torch
        r = copy.copy(self)
        r.mem = torch.empty_like(self.mem)
        base = (r.mem.data_ptr() + 255) // 256 * 256
        r.cache = lca_cache()
        lca_cache_bind(self.desc, r.cache, base, self.cache_bytes, self.batch, self.max_ctx, self.ring, stream)
        src = (self.mem.data_ptr() + 255) // 256 * 256
        o_src, o_dst = src - self.mem.data_ptr(), base - r.mem.data_ptr()
        with torch.cuda.stream(torch.cuda.ExternalStream(stream)) if stream else torch.cuda.stream(None):
            r.mem[o_dst:o_dst + self.cache_bytes].copy_(self.mem[o_src:o_src + self.cache_bytes])
        r.cache.len, r.cache.pending, r.cache.ragged = self.cache.len, self.cache.pending, self.cache.ragged
        return r

    def reset(self, stream=None):
        """Empty the cache (rebind: zeroed, len = 0) and re-zero the workspace."""
        base = (self.mem.data_ptr() + 255) // 256 * 256
        lca_cache_bind(self.desc, self.cache, base, self.cache_bytes, self.batch, self.max_ctx, self.ring, stream)
        lca_workspace_init(self.ws, self.ws_bytes, stream)

    @property
    def len(self):
        return self.cache.len

    @property
    def csa(self):
        return self.desc.kind == LCA_KIND_CSA

    @property
    def swa(self):
        return self.desc.kind == LCA_KIND_SWA

    def compress(self, kv, gate, bias, ik=None, ig=None, idx_bias=None, stream=None):
        T = kv.shape[1]
        if self.swa:
            raise ValueError("a window-only layer has no compressor: call append() alone")
        if self.csa:
            lca_csa_compress(self.cache, kv, gate, ik, ig, bias, idx_bias, T, stream)
        else:
            lca_hca_compress(self.cache, kv, gate, bias, T, stream)

    def append(self, kv, gate, ik=None, ig=None, stream=None):
        lca_swa_tail_append(self.cache, kv, gate, ik, ig, kv.shape[1], stream)

    def indexer_topk(self, qI, w, topk, stream=None):
        lca_csa_indexer_topk(self.cache, qI, w, qI.shape[1], topk, self.ws, self.ws_bytes, stream)

    def index_score(self, qI, w, stream=None):
        lca_csa_index_score(self.cache, qI, w, qI.shape[1], self.ws, self.ws_bytes, stream)

    def topk_select(self, Tq, topk, stream=None):
        lca_csa_topk_select(self.cache, Tq, topk, self.ws, self.ws_bytes, stream)

    def sparse_attn(self, q, topk, out, lse=None, stream=None):
        lca_csa_sparse_attn(self.cache, q, topk, q.shape[1], out, lse, self.ws, self.ws_bytes, stream)

    def dense_attn(self, q, out, lse=None, stream=None):
        lca_hca_dense_attn(self.cache, q, q.shape[1], out, lse, self.ws, self.ws_bytes, stream)

    def swa_attn(self, q, out, lse=None, stream=None):
        lca_swa_attn(self.cache, q, q.shape[1], out, lse, self.ws, self.ws_bytes, stream)

    def attend(self, qI, w, q, out, lse=None, topk=None, stream=None):
        lca_csa_attend(self.cache, qI, w, q, q.shape[1], topk, out, lse, self.ws, self.ws_bytes, stream)

    def topk_attn(self, q, out, lse=None, topk=None, stream=None):
        lca_csa_topk_attn(self.cache, q, q.shape[1], topk, out, lse, self.ws, self.ws_bytes, stream)

    def step(self, kv, gate, ik, ig, bias, idx_bias, qI, w, q, out, lse=None, topk=None, stream=None):
        """One decode step (CSA): T = kv.shape[1] tokens in, their queries attend."""
        lca_csa_step(self.cache, kv, gate, ik, ig, bias, idx_bias, kv.shape[1], qI, w, q, topk, out, lse, self.ws,
                     self.ws_bytes, stream)

    def hca_step(self, kv, gate, bias, q, out, lse=None, stream=None):
        """One decode step (HCA): T = kv.shape[1] tokens in (compress, append), their queries attend."""
        lca_hca_step(self.cache, kv, gate, bias, kv.shape[1], q, out, lse, self.ws, self.ws_bytes, stream)

    def swa_step(self, kv, q, out, lse=None, stream=None):
        """One decode step (window-only): T = kv.shape[1] tokens' window entries, their queries attend."""
        lca_swa_step(self.cache, kv, kv.shape[1], q, out, lse, self.ws, self.ws_bytes, stream)

    # ---- persistence: snapshots are device buffers; files hold their bytes as they are
    def snapshot(self, seq=0, stream=None):
        """Sequence `seq`'s state -> (uint8 device tensor whose first 256-aligned byte starts the
        snapshot, its lca_snapshot_info)."""
        import torch
        info = lca_snapshot_layout(self.cache)
        buf = torch.empty(info.bytes + 256, dtype=torch.uint8, device=self.mem.device)
        off = (-buf.data_ptr()) % 256
        view = buf[off:off + info.bytes]
        info = lca_cache_snapshot(self.cache, seq, view.data_ptr(), info.bytes, stream)
        return view, info

    def restore(self, snap, info, seq=-1, stream=None):
        """Restore a snapshot (device tensor from snapshot() or load_snapshot()) into sequence `seq`
        (-1: every sequence)."""
        lca_cache_restore(self.cache, seq, snap.data_ptr(), snap.numel(), info, stream)

    # ---- ragged batches: the caller's per-sequence lengths travel with every call
    def _ragged_arrays(self, lens, T):
        import numpy as np
        import torch
        lh = np.ascontiguousarray(lens, dtype=np.int64)
        th = np.ascontiguousarray(T, dtype=np.int32)
        assert lh.shape == (self.batch,) and th.shape == (self.batch,)
        ld = torch.from_numpy(lh).to(self.mem.device)
        td = torch.from_numpy(th).to(self.mem.device)
        return lh, th, ld, td

    def ragged_ingest(self, lens, T, kv, gate=None, bias=None, ik=None, ig=None, idx_bias=None, stream=None):
        """Sequence b (holding lens[b] tokens) adds the T[b] tokens in rows 0..T[b]-1 of kv[b] etc."""
        lh, th, ld, td = self._ragged_arrays(lens, T)
        lca_ragged_ingest(self.cache, kv.shape[1], lh, th, ld, td, kv, gate, ik, ig, bias, idx_bias, stream)
        import torch
        torch.cuda.current_stream().synchronize()  # the device copies of the arrays live until here

    def ragged_step(self, lens, T, kv, q, out, gate=None, bias=None, ik=None, ig=None, idx_bias=None, qI=None, w=None,
                    topk=None, lse=None, stream=None):
        """One continuous-batching step: sequence b adds T[b] tokens and their queries attend."""
        lh, th, ld, td = self._ragged_arrays(lens, T)
        lca_ragged_step(self.cache, kv.shape[1], lh, th, ld, td, kv, gate, ik, ig, bias, idx_bias, qI, w, q, topk,
                        out, lse, self.ws, self.ws_bytes, stream)
        import torch
        torch.cuda.current_stream().synchronize()

    def ragged_snapshot(self, seq, length, stream=None):
        import torch
        info = lca_ragged_snapshot(self.cache, seq, length, None, 0)
        buf = torch.empty(info.bytes + 256, dtype=torch.uint8, device=self.mem.device)
        off = (-buf.data_ptr()) % 256
        view = buf[off:off + info.bytes]
        info = lca_ragged_snapshot(self.cache, seq, length, view.data_ptr(), info.bytes, stream)
        return view, info

    def index_scores(self, Tq):
        """fp32 scores the last index_score / indexer_topk call left in the workspace: [B][Tq][max_blocks]."""
        import numpy as np
        nb = self.cache.max_blocks
        rows = []
        for qi in range(self.batch * Tq):
            off = lca_workspace_scores_offset(self.desc, self.batch, qi, self.max_ctx)
            base = self.ws - self.ws_mem.data_ptr() + off
            rows.append(self.ws_mem[base:base + nb * 4])
        import torch
        k = torch.stack(rows).cpu().numpy().view(np.uint32).reshape(self.batch, Tq, nb)
        bits = np.where(k & 0x80000000, k ^ 0x80000000, ~k).astype(np.uint32)
        return bits.view(np.float32)

    def views(self):
        """Typed torch views of the cache arrays (for checks)."""
        import torch
        c = self.cache
        B, NB, R = self.batch, c.max_blocks, self.ring
        base = self.mem.data_ptr()

        def view(addr, n, dtype, shape):
            off = addr - base
            esz = torch.tensor([], dtype=dtype).element_size()
            return self.mem[off:off + n * esz].view(dtype).view(*shape)

        v = {
            "win_codes": view(c.win_codes_dev, B * R * 64, torch.uint8, (B, R, 64)),
            "win_scale": view(c.win_scale_dev, B * R, torch.float32, (B, R)),
            "win_rope": view(c.win_rope_dev, B * R * 64, torch.int16, (B, R, 64)),
        }
        if not self.swa:
            v["blk_codes"] = view(c.blk_codes_dev, B * NB * 64, torch.uint8, (B, NB, 64))
            v["blk_scale"] = view(c.blk_scale_dev, B * NB, torch.float32, (B, NB))
            v["blk_rope"] = view(c.blk_rope_dev, B * NB * 64, torch.int16, (B, NB, 64))
        if self.csa:
            v["idx_codes"] = view(c.idx_codes_dev, B * NB * 32, torch.uint8, (B, NB, 32))
            v["idx_scale"] = view(c.idx_scale_dev, B * NB * 2, torch.uint8, (B, NB, 2))
        return v


# ----------------------------------------------------------------- snapshot files
def save_snapshot(path, snap):
    """Write a snapshot's bytes (header included) to `path`."""
    import torch
    torch.cuda.synchronize()
    snap.cpu().numpy().tofile(path)


def load_snapshot(path, device="cuda"):
    """Read a snapshot file -> (device tensor, 256-byte aligned, lca_snapshot_info from its header)."""
    import numpy as np
    import torch
    raw = np.fromfile(path, dtype=np.uint8)
    if raw.size < LCA_SNAPSHOT_HEADER:
        raise ValueError(f"{path}: {raw.size} bytes, shorter than a snapshot header")
    info = lca_snapshot_info.from_buffer_copy(raw[:ctypes.sizeof(lca_snapshot_info)].tobytes())
    if info.bytes != raw.size:
        raise ValueError(f"{path}: header says {info.bytes} bytes, file has {raw.size}")
    buf = torch.empty(raw.size + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    view = buf[off:off + raw.size]
    view.copy_(torch.from_numpy(raw))
    return view, info
