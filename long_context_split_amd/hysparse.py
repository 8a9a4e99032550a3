"""Python binding of libhysparse (ctypes): argument marshalling only.

Every step of the path runs in the HIP kernels behind the C ABI declared in
include/hysparse.h; PyTorch only provides device memory and the stream.  There
is no fallback: if libhysparse.so is not built, importing this module raises.
"""

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# HYSPARSE_LIB selects another build of the same library (the host-sanitized one in the tests)
LIB_PATH = os.environ.get("HYSPARSE_LIB") or os.path.join(_HERE, "libhysparse.so")

HS_OK, HS_ERR_INVALID_ARGUMENT, HS_ERR_UNSUPPORTED, HS_ERR_WORKSPACE_TOO_SMALL, HS_ERR_HIP = range(5)
HS_F32, HS_BF16, HS_FP8_E4M3 = 0, 1, 2
ABI_VERSION = 3


class HsError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{status_string(status)}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m long_context_split_amd.build` "
                          "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    return lib


lib = _load()


class hs_kv_cache(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("head_dim", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("capacity_rows", ctypes.c_int64),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("d_row_start", ctypes.c_void_p),
        ("h_row_start", ctypes.POINTER(ctypes.c_int64)),
        ("d_seq_len", ctypes.c_void_p),
        ("h_seq_len", ctypes.POINTER(ctypes.c_int32)),
    ]


class hs_attn_params(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("q_tokens", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("select_block", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_KVP = ctypes.POINTER(hs_kv_cache)
_PP = ctypes.POINTER(hs_attn_params)
lib.hs_abi_version.restype = ctypes.c_int
lib.hs_status_string.restype = ctypes.c_char_p
lib.hs_status_string.argtypes = [ctypes.c_int]
lib.hs_last_error.restype = ctypes.c_char_p
lib.hs_full_attn_select_workspace_size.restype = ctypes.c_size_t
lib.hs_full_attn_select_workspace_size.argtypes = [_KVP, _PP]
lib.hs_sparse_attn_workspace_size.restype = ctypes.c_size_t
lib.hs_sparse_attn_workspace_size.argtypes = [_KVP, _PP]
lib.hs_select_workspace_size.restype = ctypes.c_size_t
lib.hs_select_workspace_size.argtypes = [ctypes.c_int32] * 6
lib.hs_full_attn_select.restype = ctypes.c_int
lib.hs_full_attn_select.argtypes = [_KVP, _PP, _P, ctypes.c_int, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.hs_sparse_attn.restype = ctypes.c_int
lib.hs_sparse_attn.argtypes = [_KVP, _PP, _P, ctypes.c_int, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.hs_sparse_attn_noalloc.restype = ctypes.c_int
lib.hs_sparse_attn_noalloc.argtypes = [_KVP, _PP, _P, ctypes.c_int, _P, _P, _P, _P]
lib.hs_swa_attn.restype = ctypes.c_int
lib.hs_swa_attn.argtypes = [_KVP, _PP, _P, ctypes.c_int, _P, _P]
lib.hs_swa_attn_out.restype = ctypes.c_int
lib.hs_swa_attn_out.argtypes = [_KVP, _PP, _P, ctypes.c_int, _P, ctypes.c_int, _P]
lib.hs_prefill_chunk.restype = ctypes.c_int
lib.hs_prefill_chunk.argtypes = [_KVP, _PP, _P, ctypes.c_int, _P, ctypes.c_int, _P, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_KVP),
                                 ctypes.c_int64, _P]
lib.hs_select_from_scores.restype = ctypes.c_int
lib.hs_select_from_scores.argtypes = [_P, _P, ctypes.POINTER(ctypes.c_int32)] + [ctypes.c_int32] * 7 + \
    [_P, _P, _P, ctypes.c_size_t, _P]
lib.hs_kv_bridge.restype = ctypes.c_int
lib.hs_kv_bridge.argtypes = [_P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_P),
                             ctypes.POINTER(_P), ctypes.POINTER(_KVP), ctypes.c_int64, _P]
lib.hs_kv_append.restype = ctypes.c_int
lib.hs_kv_append.argtypes = [_P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_P),
                             ctypes.POINTER(_P), ctypes.POINTER(_KVP), _P, ctypes.POINTER(ctypes.c_int64), _P,
                             ctypes.c_size_t, _P]
lib.hs_kv_append_workspace_size.restype = ctypes.c_size_t
lib.hs_kv_append_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]

class hs_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("ms", ctypes.c_float)]


lib.hs_e4m3_check.restype = ctypes.c_int
lib.hs_e4m3_check.argtypes = [_P, _P]
lib.hs_read_probe.restype = ctypes.c_int
lib.hs_read_probe.argtypes = [_P, ctypes.c_size_t, ctypes.c_int, ctypes.c_int32, _P, _P]
lib.hs_timing_enable.restype = None
lib.hs_timing_enable.argtypes = [ctypes.c_int]
lib.hs_timing_collect.restype = ctypes.c_int
lib.hs_timing_collect.argtypes = [ctypes.POINTER(hs_kernel_time), ctypes.c_int]

if lib.hs_abi_version() != ABI_VERSION:
    raise ImportError(f"libhysparse ABI {lib.hs_abi_version()} != binding ABI {ABI_VERSION}")


def status_string(s):
    return lib.hs_status_string(int(s)).decode()


def last_error():
    return lib.hs_last_error().decode()


def check(status):
    if status != HS_OK:
        raise HsError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def cache_dtype(t):
    if t.dtype == torch.float32:
        return HS_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return HS_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return HS_FP8_E4M3
    raise TypeError(f"unsupported cache tensor dtype {t.dtype}")


def query_dtype(t):
    if t.dtype == torch.float32:
        return HS_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return HS_BF16
    raise TypeError(f"unsupported query tensor dtype {t.dtype}")


class KVCache:
    """One shared KV cache: k, v [capacity, n_kv, 128] device tensors
    (float32, bf16 or uint8 E4M3 codes with float32 k_scale / v_scale [capacity, n_kv]),
    and the rows [row_start[b], row_start[b] + seq_len[b]) of each sequence."""

    def __init__(self, k, v, seq_len=None, row_start=None, k_scale=None, v_scale=None):
        if k.shape != v.shape or k.dim() != 3 or k.shape[2] != 128:
            raise ValueError("k/v must both be [capacity, n_kv, 128]")
        if not (k.is_contiguous() and v.is_contiguous()):
            raise ValueError("k/v must be contiguous")
        self.k, self.v, self.k_scale, self.v_scale = k, v, k_scale, v_scale
        self.dtype = cache_dtype(k)
        self.capacity = k.shape[0]
        self.n_kv = k.shape[1]
        self.set_rows(seq_len, row_start)

    def set_rows(self, seq_len, row_start=None):
        if seq_len is None:
            self.batch = 0
            self.h_seq = np.zeros(1, np.int32)
            self.h_start = np.zeros(1, np.int64)
            self.d_seq = self.d_start = None
        else:
            self.h_seq = np.ascontiguousarray(np.asarray(seq_len, np.int32))
            if row_start is None:
                row_start = np.concatenate([[0], np.cumsum(self.h_seq)[:-1]])
            self.h_start = np.ascontiguousarray(np.asarray(row_start, np.int64))
            self.batch = len(self.h_seq)
            dev = self.k.device
            self.d_seq = torch.from_numpy(self.h_seq).to(dev)
            self.d_start = torch.from_numpy(self.h_start).to(dev)
        self._c = hs_kv_cache(
            self.dtype, 128, self.n_kv, self.batch, self.capacity,
            self.k.data_ptr(), self.v.data_ptr(),
            None if self.k_scale is None else self.k_scale.data_ptr(),
            None if self.v_scale is None else self.v_scale.data_ptr(),
            None if self.d_start is None else self.d_start.data_ptr(),
            self.h_start.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            None if self.d_seq is None else self.d_seq.data_ptr(),
            self.h_seq.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        )

    @property
    def c(self):
        return ctypes.byref(self._c)

    @property
    def max_len(self):
        return int(self.h_seq.max())


def params(num_q_heads, q_tokens, top_k=1024, window=128, softmax_scale=0.0, select_block=0):
    return hs_attn_params(num_q_heads, q_tokens, top_k, window, softmax_scale, select_block)


def full_attn_select_workspace_size(kv, p):
    return lib.hs_full_attn_select_workspace_size(kv.c, ctypes.byref(p))


def sparse_attn_workspace_size(kv, p):
    return lib.hs_sparse_attn_workspace_size(kv.c, ctypes.byref(p))


def workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def scores_stride(kv, window):
    return int(max(int(L) - min(window, int(L)) for L in kv.h_seq))


def full_attn_select(kv, q, top_k=1024, window=128, softmax_scale=0.0, out=None, lse=None,
                     sel_idx=None, sel_count=None, scores_out=None, ws=None, stream=None, select_block=0):
    """Full-attention layer + selection.  q [B, n_q, H, 128] (float32 or bf16).
    select_block 64 picks whole 64-token blocks (the earlier block-level variant).
    Returns (out, lse, sel_idx, sel_count) as device tensors."""
    B, n_q, H, d = q.shape
    p = params(H, n_q, top_k, window, softmax_scale, select_block)
    dev = q.device
    if out is None:
        out = torch.empty((B, n_q, H, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, H), dtype=torch.float32, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty((B, n_q, kv.n_kv, top_k + window), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((B, n_q, kv.n_kv), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(full_attn_select_workspace_size(kv, p), dev)
    check(lib.hs_full_attn_select(kv.c, ctypes.byref(p), _ptr(q), query_dtype(q), _ptr(out), _ptr(lse),
                                  _ptr(sel_idx), _ptr(sel_count), _ptr(scores_out), _ptr(ws), ws.numel(),
                                  _stream(stream)))
    return out, lse, sel_idx, sel_count


def sparse_attn(kv, q, sel_idx, sel_count, top_k=1024, window=128, softmax_scale=0.0, out=None, ws=None,
                stream=None):
    """Sparse layer over the selection of a full layer.  Returns out [B, n_q, H, 128] float32."""
    B, n_q, H, d = q.shape
    p = params(H, n_q, top_k, window, softmax_scale)
    dev = q.device
    if out is None:
        out = torch.empty((B, n_q, H, d), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(sparse_attn_workspace_size(kv, p), dev)
    check(lib.hs_sparse_attn(kv.c, ctypes.byref(p), _ptr(q), query_dtype(q), _ptr(sel_idx), _ptr(sel_count),
                             _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def sparse_attn_noalloc(kv, q, sel_idx, sel_count, top_k=1024, window=128, softmax_scale=0.0, out=None,
                        stream=None):
    """hs_sparse_attn_noalloc: the sparse layer with its scratch in the library's static device array
    (no workspace).  out must be given by callers that cannot allocate."""
    B, n_q, H, d = q.shape
    p = params(H, n_q, top_k, window, softmax_scale)
    if out is None:
        out = torch.empty((B, n_q, H, d), dtype=torch.float32, device=q.device)
    check(lib.hs_sparse_attn_noalloc(kv.c, ctypes.byref(p), _ptr(q), query_dtype(q), _ptr(sel_idx),
                                     _ptr(sel_count), _ptr(out), _stream(stream)))
    return out


def _out_dtype(t):
    if t.dtype == torch.float32:
        return HS_F32
    if t.dtype == torch.bfloat16:
        return HS_BF16
    raise TypeError(f"unsupported output tensor dtype {t.dtype}")


def swa_attn(kv, q, window, softmax_scale=0.0, out=None, out_dtype=torch.float32, stream=None):
    """Sliding-window attention of the last q_tokens cache rows of every sequence (band of `window`
    rows ending at each query's own row).  Returns out [B, n_q, H, 128], float32 or bf16 (the dtype of
    a given `out`, else `out_dtype`)."""
    B, n_q, H, d = q.shape
    p = params(H, n_q, 0, window, softmax_scale)
    if out is None:
        out = torch.empty((B, n_q, H, d), dtype=out_dtype, device=q.device)
    check(lib.hs_swa_attn_out(kv.c, ctypes.byref(p), _ptr(q), query_dtype(q), _ptr(out), _out_dtype(out),
                              _stream(stream)))
    return out


def select_from_scores(scores, seq_len, q_tokens, n_kv, top_k=1024, window=128, select_block=0, stream=None):
    """Selection stage alone on given float32 scores [B, q_tokens, n_kv, S]."""
    h_seq = np.ascontiguousarray(np.asarray(seq_len, np.int32))
    B = len(h_seq)
    max_len = int(h_seq.max())
    dev = scores.device
    d_seq = torch.from_numpy(h_seq).to(dev)
    sel_idx = torch.empty((B, q_tokens, n_kv, top_k + window), dtype=torch.int32, device=dev)
    sel_count = torch.empty((B, q_tokens, n_kv), dtype=torch.int32, device=dev)
    ws = workspace(lib.hs_select_workspace_size(B, q_tokens, n_kv, max_len, top_k, window), dev)
    check(lib.hs_select_from_scores(_ptr(scores), _ptr(d_seq), h_seq.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                    B, q_tokens, n_kv, max_len, top_k, window, select_block, _ptr(sel_idx),
                                    _ptr(sel_count),
                                    _ptr(ws), ws.numel(), _stream(stream)))
    return sel_idx, sel_count


def kv_bridge(hidden, w_k, w_v, targets, row_offset, stream=None):
    """KV Bridging: hidden [T, Dm] bf16; w_k/w_v lists of [Dm, 128] bf16; targets list of KVCache."""
    n = len(targets)
    wk = (ctypes.c_void_p * n)(*[w.data_ptr() for w in w_k])
    wv = (ctypes.c_void_p * n)(*[w.data_ptr() for w in w_v])
    tg = (_KVP * n)(*[ctypes.pointer(t._c) for t in targets])
    check(lib.hs_kv_bridge(_ptr(hidden), hidden.shape[0], hidden.shape[1], n, wk, wv, tg, int(row_offset),
                           _stream(stream)))


def prefill_chunk(self_kv, q, window, hidden, w_k, w_v, targets, row_offset, swa_out=None, softmax_scale=0.0,
                  swa_out_dtype=torch.float32, stream=None):
    """One Self-Decoder prefill chunk: sliding-window attention of the chunk's queries q [1, T, H, 128]
    (the chunk's rows are the last T rows of self_kv) and KV Bridging of its hidden states [T, Dm] into
    every target at rows [row_offset, row_offset + T).  Returns the attention output [1, T, H, 128]."""
    B, T, H, d = q.shape
    p = params(H, T, 0, window, softmax_scale)
    if swa_out is None:
        swa_out = torch.empty((B, T, H, d), dtype=swa_out_dtype, device=q.device)
    n = len(targets)
    wk = (ctypes.c_void_p * n)(*[w.data_ptr() for w in w_k])
    wv = (ctypes.c_void_p * n)(*[w.data_ptr() for w in w_v])
    tg = (_KVP * n)(*[ctypes.pointer(t._c) for t in targets])
    check(lib.hs_prefill_chunk(self_kv.c, ctypes.byref(p), _ptr(q), query_dtype(q), _ptr(swa_out), _out_dtype(swa_out),
                               _ptr(hidden),
                               hidden.shape[0], hidden.shape[1], n, wk, wv, tg, int(row_offset), _stream(stream)))
    return swa_out


def kv_append_workspace_size(n_tokens, d_model, n_targets):
    return lib.hs_kv_append_workspace_size(n_tokens, d_model, n_targets)


def kv_append(hidden, w_k, w_v, targets, rows, ws=None, stream=None):
    """Decode-time append: token t of hidden [n, Dm] bf16 goes to cache row rows[t] of every target.
    rows: int64 sequence or device tensor; both a device and a host copy are passed."""
    h_rows = np.ascontiguousarray(np.asarray(rows.cpu() if isinstance(rows, torch.Tensor) else rows, np.int64))
    d_rows = torch.from_numpy(h_rows).to(hidden.device)
    n = len(targets)
    if ws is None:
        ws = workspace(kv_append_workspace_size(hidden.shape[0], hidden.shape[1], n), hidden.device)
    wk = (ctypes.c_void_p * n)(*[w.data_ptr() for w in w_k])
    wv = (ctypes.c_void_p * n)(*[w.data_ptr() for w in w_v])
    tg = (_KVP * n)(*[ctypes.pointer(t._c) for t in targets])
    check(lib.hs_kv_append(_ptr(hidden), hidden.shape[0], hidden.shape[1], n, wk, wv, tg, _ptr(d_rows),
                           h_rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ptr(ws), ws.numel(),
                           _stream(stream)))
    return d_rows


def read_probe(buf, nbytes=None, non_temporal=True, grid=256, sink=None, stream=None):
    """Streaming read of a device tensor's first nbytes (the measured-peak probe)."""
    nbytes = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    if sink is None:
        sink = torch.empty(4, dtype=torch.int32, device=buf.device)
    check(lib.hs_read_probe(_ptr(buf), nbytes, 1 if non_temporal else 0, grid, _ptr(sink), _stream(stream)))


def e4m3_check(stream=None):
    """hs_e4m3_check: (mismatches, values compared) of the library's hardware E4M3 conversion against
    the bit-level RNE reference over every finite float32 with |y| < 464."""
    counts = torch.empty(2, dtype=torch.int64, device="cuda")
    check(lib.hs_e4m3_check(_ptr(counts), _stream(stream)))
    c = counts.cpu().tolist()
    return int(c[0]), int(c[1])


def timing_enable(on=True):
    """Bracket every library launch with HIP events on its stream (profiling aid)."""
    lib.hs_timing_enable(1 if on else 0)


def timing_collect(max_records=1 << 16):
    """[(kernel name, ms), ...] of the launches recorded since the last collect."""
    buf = (hs_kernel_time * max_records)()
    n = lib.hs_timing_collect(buf, max_records)
    if n < 0:
        raise HsError(HS_ERR_HIP, "event timing failed")
    return [(buf[i].name.decode(), float(buf[i].ms)) for i in range(n)]
