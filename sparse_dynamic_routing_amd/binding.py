"""ctypes binding of libgm.so, the C ABI declared in include/gm.h.

Argument marshalling only: every function here checks that the torch
tensors it is given match the C call (device, dtype, contiguity, shapes),
then passes their device pointers, sizes and the current HIP stream to the
library.  All arithmetic runs in the HIP kernels.  There is no fallback: if
libgm.so is missing or cannot be loaded, every call raises.

The functions named like the C calls (``gm_ser_forward`` ...) write into
output tensors the caller provides; ``ser_forward`` and friends allocate the
outputs with torch and return them.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgm.so")

GM_F32, GM_BF16 = 0, 1
STATUS = {0: "GM_OK", 1: "GM_ERR_NULL", 2: "GM_ERR_SHAPE", 3: "GM_ERR_UNSUPPORTED",
          4: "GM_ERR_WORKSPACE", 5: "GM_ERR_HIP", 6: "GM_ERR_ALIGN", 7: "GM_ERR_ALIAS",
          8: "GM_ERR_TOO_LARGE"}
EXPORTS = ("gm_ser_forward", "gm_ser_forward_chain2", "gm_sea_forward", "gm_sea_backward_workspace_bytes",
           "gm_sea_backward", "gm_sea_backward_noalloc", "gm_ser_sea_forward", "gm_decode_step", "gm_dense_refresh", "gm_leg_mix_forward",
           "gm_leg_mix_backward_workspace_bytes", "gm_leg_mix_backward",
           "gm_ser_backward_workspace_bytes", "gm_ser_backward", "gm_check_edges",
           "gm_status_string", "gm_abi_version")


class GMError(RuntimeError):
    def __init__(self, call: str, code: int, text: str):
        super().__init__(f"{call} failed: {STATUS.get(code, code)} ({text})")
        self.code = code


_lib = None
_I, _P, _F, _Z = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgm.so (torch first, so the library binds to torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m sparse_dynamic_routing_amd.build`")
    lib = ctypes.CDLL(path)
    sig = {
        "gm_ser_forward": [_I, _I, _I, _P, _P, _I, _P, _P, _I, _P, _P, _I, _P, _P],
        "gm_ser_forward_chain2": [_I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P],
        "gm_sea_forward": [_I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _I, _P, _P, _P],
        "gm_sea_backward_workspace_bytes": [_I, _I, _I, _I, _I],
        "gm_sea_backward": [_I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _I, _P, _P,
                            _P, _P, _P, _P, _P, _Z, _P],
        "gm_sea_backward_noalloc": [_I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _I, _P,
                                    _P, _P, _P, _P, _P, _P],
        "gm_ser_sea_forward": [_I, _I, _I, _I, _I, _I, _F, _P, _P, _I, _P, _P, _I, _I, _P, _P,
                               _P, _P, _P, _P, _P, _P, _P],
        "gm_decode_step": [_I, _I, _I, _I, _I, _I, _F, _P, _P, _I, _P, _P, _I, _I, _P, _P,
                           _P, _P, _P, _P, _P],
        "gm_dense_refresh": [_I, _I, _I, _I, _I, _I, _F, _P, _P, _I, _I, _P, _P, _P, _P],
        "gm_leg_mix_forward": [_I, _I, _I, _P, _P, _I, _P, _I, _P, _P, _P],
        "gm_leg_mix_backward_workspace_bytes": [_I, _I, _I, _I],
        "gm_leg_mix_backward": [_I, _I, _I, _P, _P, _I, _P, _P, _P, _I, _P, _P, _P, _P, _Z,
                                _P],
        "gm_ser_backward_workspace_bytes": [_I, _I, _I, _I, _I, _I],
        "gm_ser_backward": [_I, _I, _I, _P, _P, _I, _P, _P, _I, _P, _P, _I, _P, _P, _P, _P,
                            _P, _Z, _P],
        "gm_check_edges": [_I, _I, _I, _P, _P, _I, _P, _P],
        "gm_status_string": [_I],
        "gm_abi_version": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = _I
    lib.gm_ser_backward_workspace_bytes.restype = _Z
    lib.gm_sea_backward_workspace_bytes.restype = _Z
    lib.gm_leg_mix_backward_workspace_bytes.restype = _Z
    lib.gm_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _call(name: str, *args) -> None:
    lib = load()
    rc = getattr(lib, name)(*args)
    if rc != 0:
        raise GMError(name, rc, lib.gm_status_string(rc).decode())


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtypes, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _act_dtype(t: torch.Tensor) -> int:
    return GM_BF16 if t.dtype == torch.bfloat16 else GM_F32


_ACT = (torch.float32, torch.bfloat16)


# --------------------------------------------------------------- C-named calls
def gm_ser_forward(idx1, w1, idx2, w2, idx_out, w_out, stream=None, paths=None) -> None:
    """``paths`` (optional, [B, n, hkv] int64) receives the path map that
    gm_ser_backward can take."""
    B, n, hkv, s2 = idx1.shape
    s3, s1 = idx2.shape[-1], idx_out.shape[-1]
    _need(idx1, "idx1", (torch.int32,)); _need(w1, "w1", (torch.float32,), idx1.shape)
    _need(idx2, "idx2", (torch.int32,), (B, n, hkv, s3))
    _need(w2, "w2", (torch.float32,), idx2.shape)
    _need(idx_out, "idx_out", (torch.int32,), (B, n, hkv, s1))
    _need(w_out, "w_out", (torch.float32,), idx_out.shape)
    if paths is not None:
        _need(paths, "paths", (torch.int64,), (B, n, hkv))
    _call("gm_ser_forward", B, n, hkv, _ptr(idx1), _ptr(w1), s2, _ptr(idx2), _ptr(w2), s3,
          _ptr(idx_out), _ptr(w_out), s1, _ptr(paths), _stream(stream))


def stats_shape(q: torch.Tensor, hkv: int, s1: int) -> tuple:
    """Shape of the saved statistics for query tensor q [B, n, hq, d]:
    [B, hkv, n, E G + 2, s1] 4-byte words, E = 1 for bf16 inputs (fp32 p / w)
    and 2 for fp32 inputs (fp64 p / w)."""
    B, n, hq, _ = q.shape
    E = 1 if q.dtype == torch.bfloat16 else 2
    return (B, hkv, n, E * (hq // hkv) + 2, s1)


def gm_sea_forward(q, k, v, idx, w, o, scale=None, stream=None, stats=None) -> None:
    """``stats`` (optional, ``stats_shape(q, hkv, s1)`` fp32 words) receives p / w
    per query head and slot, then a copy of the edge indices (int32 bits) and
    weights, for gm_sea_backward."""
    B, n, hq, d = q.shape
    hkv, s1 = idx.shape[2], idx.shape[3]
    _need(q, "q", _ACT)
    _need(k, "k", (q.dtype,), (B, n, hkv, d)); _need(v, "v", (q.dtype,), (B, n, hkv, d))
    _need(idx, "idx", (torch.int32,), (B, n, hkv, s1)); _need(w, "w", (torch.float32,), idx.shape)
    _need(o, "o", (q.dtype,), q.shape)
    if stats is not None:
        _need(stats, "stats", (torch.float32,), stats_shape(q, hkv, s1))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _call("gm_sea_forward", B, n, hq, hkv, d, _act_dtype(q), scale, _ptr(q), _ptr(k), _ptr(v),
          _ptr(idx), _ptr(w), s1, _ptr(o), _ptr(stats), _stream(stream))


def gm_ser_sea_forward(idx1, w1, idx2, w2, q, k, v, idx_out, w_out, o, scale=None, stream=None,
                       stats=None, paths=None) -> None:
    """SER (A' into idx_out / w_out) then SEA (o, and stats when given) in
    one call."""
    B, n, hkv, s2 = idx1.shape
    s3, s1 = idx2.shape[3], idx_out.shape[3]
    hq, d = q.shape[2], q.shape[3]
    _need(idx1, "idx1", (torch.int32,)); _need(w1, "w1", (torch.float32,), idx1.shape)
    _need(idx2, "idx2", (torch.int32,), (B, n, hkv, s3)); _need(w2, "w2", (torch.float32,), idx2.shape)
    _need(idx_out, "idx_out", (torch.int32,), (B, n, hkv, s1))
    _need(w_out, "w_out", (torch.float32,), idx_out.shape)
    _need(q, "q", _ACT, (B, n, hq, d))
    _need(k, "k", (q.dtype,), (B, n, hkv, d)); _need(v, "v", (q.dtype,), (B, n, hkv, d))
    _need(o, "o", (q.dtype,), q.shape)
    if stats is not None:
        _need(stats, "stats", (torch.float32,), stats_shape(q, hkv, s1))
    if paths is not None:
        _need(paths, "paths", (torch.int64,), (B, n, hkv))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _call("gm_ser_sea_forward", B, n, hq, hkv, d, _act_dtype(q), scale, _ptr(idx1), _ptr(w1), s2,
          _ptr(idx2), _ptr(w2), s3, s1, _ptr(q), _ptr(k), _ptr(v), _ptr(idx_out), _ptr(w_out),
          _ptr(o), _ptr(stats), _ptr(paths), _stream(stream))


def gm_sea_backward_workspace_bytes(B, n, hq, hkv, s1) -> int:
    return int(load().gm_sea_backward_workspace_bytes(B, n, hq, hkv, s1))


def gm_sea_backward(q, k, v, idx, w, dout, dq, dk, dv, dw, workspace, scale=None,
                    stream=None, stats=None) -> None:
    """``stats``: optional, what gm_sea_forward wrote for the same inputs."""
    B, n, hq, d = q.shape
    hkv, s1 = idx.shape[2], idx.shape[3]
    _need(q, "q", _ACT)
    _need(k, "k", (q.dtype,), (B, n, hkv, d)); _need(v, "v", (q.dtype,), (B, n, hkv, d))
    _need(idx, "idx", (torch.int32,), (B, n, hkv, s1)); _need(w, "w", (torch.float32,), idx.shape)
    _need(dout, "dout", (q.dtype,), q.shape)
    _need(dq, "dq", (torch.float32,), q.shape)
    _need(dk, "dk", (torch.float32,), k.shape); _need(dv, "dv", (torch.float32,), v.shape)
    _need(dw, "dw", (torch.float32,), idx.shape)
    _need(workspace, "workspace", (torch.uint8, torch.float64))
    if stats is not None:
        _need(stats, "stats", (torch.float32,), stats_shape(q, hkv, s1))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _call("gm_sea_backward", B, n, hq, hkv, d, _act_dtype(q), scale, _ptr(q), _ptr(k), _ptr(v),
          _ptr(idx), _ptr(w), s1, _ptr(dout), _ptr(stats), _ptr(dq), _ptr(dk), _ptr(dv),
          _ptr(dw), _ptr(workspace), workspace.numel() * workspace.element_size(),
          _stream(stream))


def gm_sea_backward_noalloc(q, k, v, idx, w, dout, dq, dk, dv, dw, scale=None, stream=None,
                            stats=None) -> None:
    """gm_sea_backward with the library's fixed per-GPU scratch instead of a
    workspace (the call allocates nothing)."""
    B, n, hq, d = q.shape
    hkv, s1 = idx.shape[2], idx.shape[3]
    _need(q, "q", _ACT)
    _need(k, "k", (q.dtype,), (B, n, hkv, d)); _need(v, "v", (q.dtype,), (B, n, hkv, d))
    _need(idx, "idx", (torch.int32,), (B, n, hkv, s1)); _need(w, "w", (torch.float32,), idx.shape)
    _need(dout, "dout", (q.dtype,), q.shape)
    _need(dq, "dq", (torch.float32,), q.shape)
    _need(dk, "dk", (torch.float32,), k.shape); _need(dv, "dv", (torch.float32,), v.shape)
    _need(dw, "dw", (torch.float32,), idx.shape)
    if stats is not None:
        _need(stats, "stats", (torch.float32,), stats_shape(q, hkv, s1))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _call("gm_sea_backward_noalloc", B, n, hq, hkv, d, _act_dtype(q), scale, _ptr(q), _ptr(k),
          _ptr(v), _ptr(idx), _ptr(w), s1, _ptr(dout), _ptr(stats), _ptr(dq), _ptr(dk),
          _ptr(dv), _ptr(dw), _stream(stream))


def gm_decode_step(idx1, w1, idx2, w2, q, k, v, idx_out, w_out, o, scale=None,
                   stream=None) -> None:
    """One decode step: idx1/w1 [B, hkv, s2] (the new tokens' leg-1 rows),
    idx2/w2 [B, T, hkv, s3] (edge cache), q [B, hq, d], k/v [B, T, hkv, d]
    -> idx_out/w_out [B, hkv, s1], o [B, hq, d]."""
    B, hkv, s2 = idx1.shape
    T, s3 = idx2.shape[1], idx2.shape[3]
    hq, d = q.shape[1], q.shape[2]
    s1 = idx_out.shape[2]
    _need(idx1, "idx1", (torch.int32,)); _need(w1, "w1", (torch.float32,), idx1.shape)
    _need(idx2, "idx2", (torch.int32,), (B, T, hkv, s3))
    _need(w2, "w2", (torch.float32,), idx2.shape)
    _need(q, "q", _ACT, (B, hq, d))
    _need(k, "k", (q.dtype,), (B, T, hkv, d)); _need(v, "v", (q.dtype,), (B, T, hkv, d))
    _need(idx_out, "idx_out", (torch.int32,), (B, hkv, s1))
    _need(w_out, "w_out", (torch.float32,), idx_out.shape)
    _need(o, "o", (q.dtype,), q.shape)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _call("gm_decode_step", B, T, hq, hkv, d, _act_dtype(q), scale, _ptr(idx1), _ptr(w1), s2,
          _ptr(idx2), _ptr(w2), s3, s1, _ptr(q), _ptr(k), _ptr(v), _ptr(idx_out), _ptr(w_out),
          _ptr(o), _stream(stream))


def gm_dense_refresh(q, k, lse, idx_out, w_out, lse_given=False, scale=None,
                     stream=None) -> None:
    """Refresh edges idx_out/w_out [B, n, hkv, s] from dense causal attention
    over q [B, n, hq, d], k [B, n, hkv, d] (bf16); lse [B, n, hq] fp32 is
    written, or read when ``lse_given``."""
    B, n, hq, d = q.shape
    hkv = k.shape[2]
    s = idx_out.shape[3]
    _need(q, "q", (torch.bfloat16,))
    _need(k, "k", (torch.bfloat16,), (B, n, hkv, d))
    _need(lse, "lse", (torch.float32,), (B, n, hq))
    _need(idx_out, "idx_out", (torch.int32,), (B, n, hkv, s))
    _need(w_out, "w_out", (torch.float32,), idx_out.shape)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _call("gm_dense_refresh", B, n, hq, hkv, d, GM_BF16, scale, _ptr(q), _ptr(k), s,
          1 if lse_given else 0, _ptr(lse), _ptr(idx_out), _ptr(w_out), _stream(stream))


def gm_leg_mix_forward(idx, w, alpha, idx_out, w_out, stream=None) -> None:
    """One leg [B, n, hkv, s] from the stored edges [B, n, hkv, K] mixed by
    alpha [hkv, K]."""
    B, n, hkv, K = idx.shape
    s = idx_out.shape[3]
    _need(idx, "idx", (torch.int32,)); _need(w, "w", (torch.float32,), idx.shape)
    _need(alpha, "alpha", (torch.float32,), (hkv, K))
    _need(idx_out, "idx_out", (torch.int32,), (B, n, hkv, s))
    _need(w_out, "w_out", (torch.float32,), idx_out.shape)
    _call("gm_leg_mix_forward", B, n, hkv, _ptr(idx), _ptr(w), K, _ptr(alpha), s,
          _ptr(idx_out), _ptr(w_out), _stream(stream))


def gm_leg_mix_backward_workspace_bytes(B, n, hkv, K) -> int:
    return int(load().gm_leg_mix_backward_workspace_bytes(B, n, hkv, K))


def gm_leg_mix_backward(idx, w, alpha, idx_out, w_out, dleg, dw, dalpha, workspace,
                        stream=None) -> None:
    B, n, hkv, K = idx.shape
    s = idx_out.shape[3]
    _need(idx, "idx", (torch.int32,)); _need(w, "w", (torch.float32,), idx.shape)
    _need(alpha, "alpha", (torch.float32,), (hkv, K))
    _need(idx_out, "idx_out", (torch.int32,), (B, n, hkv, s))
    _need(w_out, "w_out", (torch.float32,), idx_out.shape)
    _need(dleg, "dleg", (torch.float32,), idx_out.shape)
    _need(dw, "dw", (torch.float32,), idx.shape); _need(dalpha, "dalpha", (torch.float32,), (hkv, K))
    _need(workspace, "workspace", (torch.uint8, torch.float64))
    _call("gm_leg_mix_backward", B, n, hkv, _ptr(idx), _ptr(w), K, _ptr(alpha), _ptr(idx_out),
          _ptr(w_out), s, _ptr(dleg), _ptr(dw), _ptr(dalpha), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(stream))


def gm_ser_backward_workspace_bytes(B, n, hkv, s2, s3, aliased) -> int:
    return int(load().gm_ser_backward_workspace_bytes(B, n, hkv, s2, s3, int(bool(aliased))))


def gm_ser_backward(idx1, w1, idx2, w2, idx_out, w_out, dw_out, dw1, dw2, workspace,
                    stream=None, paths=None) -> None:
    """``paths``: optional, the map gm_ser_forward wrote for the same legs."""
    B, n, hkv, s2 = idx1.shape
    s3, s1 = idx2.shape[-1], idx_out.shape[-1]
    _need(idx1, "idx1", (torch.int32,)); _need(w1, "w1", (torch.float32,), idx1.shape)
    _need(idx2, "idx2", (torch.int32,), (B, n, hkv, s3))
    _need(w2, "w2", (torch.float32,), idx2.shape)
    _need(idx_out, "idx_out", (torch.int32,), (B, n, hkv, s1))
    _need(w_out, "w_out", (torch.float32,), idx_out.shape)
    _need(dw_out, "dw_out", (torch.float32,), idx_out.shape)
    _need(dw1, "dw1", (torch.float32,), idx1.shape); _need(dw2, "dw2", (torch.float32,), idx2.shape)
    _need(workspace, "workspace", (torch.uint8, torch.float64))
    if paths is not None:
        _need(paths, "paths", (torch.int64,), (B, n, hkv))
    _call("gm_ser_backward", B, n, hkv, _ptr(idx1), _ptr(w1), s2, _ptr(idx2), _ptr(w2), s3,
          _ptr(idx_out), _ptr(w_out), s1, _ptr(dw_out), _ptr(paths), _ptr(dw1), _ptr(dw2),
          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))


def gm_ser_forward_chain2(idx, w, idx_out, w_out, idx_mid=None, w_mid=None,
                          stream=None) -> None:
    """Two chained referral steps: A2 -> (idx_out, w_out), A1 -> (idx_mid,
    w_mid) when given."""
    B, n, hkv, s = idx.shape
    _need(idx, "idx", (torch.int32,)); _need(w, "w", (torch.float32,), idx.shape)
    _need(idx_out, "idx_out", (torch.int32,), idx.shape)
    _need(w_out, "w_out", (torch.float32,), idx.shape)
    if idx_mid is not None:
        _need(idx_mid, "idx_mid", (torch.int32,), idx.shape)
    if w_mid is not None:
        _need(w_mid, "w_mid", (torch.float32,), idx.shape)
    _call("gm_ser_forward_chain2", B, n, hkv, _ptr(idx), _ptr(w), s, _ptr(idx_mid),
          _ptr(w_mid), _ptr(idx_out), _ptr(w_out), _stream(stream))


def gm_check_edges(idx, w, counts, stream=None) -> None:
    B, n, hkv, s = idx.shape
    _need(idx, "idx", (torch.int32,)); _need(w, "w", (torch.float32,), idx.shape)
    _need(counts, "counts", (torch.int64,), (2,))
    _call("gm_check_edges", B, n, hkv, _ptr(idx), _ptr(w), s, _ptr(counts), _stream(stream))


# ------------------------------------------------------- allocating wrappers
def ser_forward(idx1, w1, idx2, w2, s1, stream=None, save_paths=False):
    """(idx_out, w_out), with ``save_paths`` also the path map."""
    shape = tuple(idx1.shape[:3]) + (s1,)
    idx_out = torch.empty(shape, dtype=torch.int32, device=idx1.device)
    w_out = torch.empty(shape, dtype=torch.float32, device=idx1.device)
    paths = (torch.empty(tuple(idx1.shape[:3]), dtype=torch.int64, device=idx1.device)
             if save_paths else None)
    gm_ser_forward(idx1, w1, idx2, w2, idx_out, w_out, stream, paths)
    return (idx_out, w_out, paths) if save_paths else (idx_out, w_out)


def ser_forward_chain2(idx, w, stream=None, save_mid=False):
    """(idx_out, w_out) of Sp(A1 A1) with A1 = Sp(A0 A0), A0 = (idx, w), in
    one call; with ``save_mid`` also (idx_mid, w_mid) = A1."""
    idx_out = torch.empty_like(idx)
    w_out = torch.empty_like(w)
    idx_mid = torch.empty_like(idx) if save_mid else None
    w_mid = torch.empty_like(w) if save_mid else None
    gm_ser_forward_chain2(idx, w, idx_out, w_out, idx_mid, w_mid, stream)
    return (idx_out, w_out, idx_mid, w_mid) if save_mid else (idx_out, w_out)


def sea_forward(q, k, v, idx, w, scale=None, stream=None, save_stats=False):
    """o, or (o, stats) with ``save_stats`` (stats ``stats_shape(q, hkv, s1)``:
    p / w per query head and slot, then the edge row, for sea_backward)."""
    o = torch.empty_like(q)
    B, n, hq, _ = q.shape
    hkv, s1 = idx.shape[2], idx.shape[3]
    stats = (torch.empty(stats_shape(q, hkv, s1), dtype=torch.float32, device=q.device)
             if save_stats else None)
    gm_sea_forward(q, k, v, idx, w, o, scale, stream, stats)
    return (o, stats) if save_stats else o


def ser_sea_forward(idx1, w1, idx2, w2, s1, q, k, v, scale=None, stream=None, save_stats=False,
                    save_paths=False):
    """(idx_out, w_out, o[, stats][, paths]) of SER then SEA in one call."""
    B, n, hkv, _ = idx1.shape
    hq = q.shape[2]
    io = torch.empty((B, n, hkv, s1), dtype=torch.int32, device=idx1.device)
    wo = torch.empty((B, n, hkv, s1), dtype=torch.float32, device=idx1.device)
    o = torch.empty_like(q)
    stats = (torch.empty(stats_shape(q, hkv, s1), dtype=torch.float32, device=q.device)
             if save_stats else None)
    paths = (torch.empty((B, n, hkv), dtype=torch.int64, device=q.device)
             if save_paths else None)
    gm_ser_sea_forward(idx1, w1, idx2, w2, q, k, v, io, wo, o, scale, stream, stats, paths)
    return (io, wo, o) + ((stats,) if save_stats else ()) + ((paths,) if save_paths else ())


def sea_workspace(q, idx, device=None) -> torch.Tensor:
    B, n, hq, _ = q.shape
    nbytes = gm_sea_backward_workspace_bytes(B, n, hq, idx.shape[2], idx.shape[3])
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device or q.device)


def sea_backward(q, k, v, idx, w, dout, scale=None, workspace=None, stream=None, stats=None):
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32)
    dk = torch.empty(k.shape, **f32)
    dv = torch.empty(v.shape, **f32)
    dw = torch.empty(idx.shape, **f32)
    ws = sea_workspace(q, idx) if workspace is None else workspace
    gm_sea_backward(q, k, v, idx, w, dout, dq, dk, dv, dw, ws, scale, stream, stats)
    return dq, dk, dv, dw


def ser_workspace(idx1, idx2, aliased, device=None) -> torch.Tensor:
    B, n, hkv, s2 = idx1.shape
    nbytes = gm_ser_backward_workspace_bytes(B, n, hkv, s2, idx2.shape[-1], aliased)
    return torch.empty(max(nbytes, 8) // 8, dtype=torch.float64,
                       device=device or idx1.device)


def ser_backward(idx1, w1, idx2, w2, idx_out, w_out, dw_out, aliased=False, workspace=None,
                 stream=None, paths=None):
    """(dw1, dw2); with ``aliased`` the legs are one tensor and one gradient
    (the same tensor, returned twice) receives both contributions."""
    dw1 = torch.empty(idx1.shape, dtype=torch.float32, device=idx1.device)
    dw2 = dw1 if aliased else torch.empty(idx2.shape, dtype=torch.float32, device=idx1.device)
    ws = ser_workspace(idx1, idx2, aliased) if workspace is None else workspace
    gm_ser_backward(idx1, w1, idx2, w2, idx_out, w_out, dw_out, dw1, dw2, ws, stream, paths)
    return dw1, dw2


def check_edges(idx, w, stream=None):
    """(bad slots, live slots) of an edge tensor; synchronises the stream."""
    counts = torch.zeros(2, dtype=torch.int64, device=idx.device)
    gm_check_edges(idx, w, counts, stream)
    c = counts.cpu()
    return int(c[0]), int(c[1])


def stats_as_query_heads(stats: torch.Tensor, G: int) -> torch.Tensor:
    """The p / w rows of the saved statistics [B, hkv, n, E G + 2, s1] of G
    query heads per KV head as [B, n, hq, s1] (fp32 for E = 1, fp64 for
    E = 2)."""
    B, hkv, n, R, s1 = stats.shape
    E = (R - 2) // G
    if E not in (1, 2) or E * G + 2 != R:
        raise ValueError(f"statistics of {R} rows do not fit G = {G}")
    pw = stats[:, :, :, :E * G].reshape(B, hkv, n, E * G * s1)
    if E == 2:
        pw = pw.contiguous().view(torch.float64)          # G s1 doubles per unit
    return pw.reshape(B, hkv, n, G, s1).permute(0, 2, 1, 3, 4).reshape(B, n, hkv * G, s1)


def stats_edge_copy(stats: torch.Tensor):
    """The edge copy in the saved statistics as (idx [B, n, hkv, s1] int32,
    w [B, n, hkv, s1] fp32)."""
    e = stats[:, :, :, -2:].permute(0, 2, 1, 3, 4)
    return e[..., 0, :].contiguous().view(torch.int32), e[..., 1, :].contiguous()


def decode_step(idx1, w1, idx2, w2, q, k, v, s1, scale=None, stream=None):
    """(idx_out, w_out, o) of one decode step (see gm_decode_step)."""
    B, hkv, _ = idx1.shape
    idx_out = torch.empty((B, hkv, s1), dtype=torch.int32, device=q.device)
    w_out = torch.empty((B, hkv, s1), dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    gm_decode_step(idx1, w1, idx2, w2, q, k, v, idx_out, w_out, o, scale, stream)
    return idx_out, w_out, o


def dense_refresh(q, k, s, lse=None, scale=None, stream=None):
    """(idx_out, w_out, lse) of the refresh edges (see gm_dense_refresh); a
    given ``lse`` (the dense layer's own) skips the first pass."""
    B, n, hq, _ = q.shape
    hkv = k.shape[2]
    idx_out = torch.empty((B, n, hkv, s), dtype=torch.int32, device=q.device)
    w_out = torch.empty((B, n, hkv, s), dtype=torch.float32, device=q.device)
    given = lse is not None
    if not given:
        lse = torch.empty((B, n, hq), dtype=torch.float32, device=q.device)
    gm_dense_refresh(q, k, lse, idx_out, w_out, given, scale, stream)
    return idx_out, w_out, lse


def leg_mix(idx, w, alpha, s, stream=None):
    """(idx_out, w_out) of one leg (see gm_leg_mix_forward)."""
    B, n, hkv, _ = idx.shape
    idx_out = torch.empty((B, n, hkv, s), dtype=torch.int32, device=idx.device)
    w_out = torch.empty((B, n, hkv, s), dtype=torch.float32, device=idx.device)
    gm_leg_mix_forward(idx, w, alpha, idx_out, w_out, stream)
    return idx_out, w_out


def leg_mix_backward(idx, w, alpha, idx_out, w_out, dleg, stream=None):
    """(dw, dalpha) of one leg (see gm_leg_mix_backward)."""
    B, n, hkv, K = idx.shape
    dw = torch.empty(idx.shape, dtype=torch.float32, device=idx.device)
    dalpha = torch.empty((hkv, K), dtype=torch.float32, device=idx.device)
    nbytes = gm_leg_mix_backward_workspace_bytes(B, n, hkv, K)
    ws = torch.empty(max(nbytes, 8) // 8, dtype=torch.float64, device=idx.device)
    gm_leg_mix_backward(idx, w, alpha, idx_out, w_out, dleg, dw, dalpha, ws, stream)
    return dw, dalpha
