"""Python binding of the CSA HIP library (``libcsa.so``, C ABI in ``include/csa.h``).

Argument marshalling only: every step of the attention path runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU; their data pointers and the current HIP
stream are passed through unchanged.  There is no CPU fallback: if the library is missing
or a call fails, an exception is raised.

The functions keep the C names: ``csa_compress``, ``csa_index_topk``, ``csa_attend``,
``csa_forward``, ``csa_workspace_size`` and friends.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "lib_path", "load", "Dims", "Cache", "Weights", "CsaError",
    "csa_abi_version", "csa_row_bytes", "csa_state_width", "csa_state_rows",
    "csa_workspace_size", "csa_compress", "csa_index_topk", "csa_attend", "csa_forward",
    "csa_index_scores", "csa_topk", "csa_topk_workspace_size", "ProjWeights", "csa_query_project",
    "csa_query_project_workspace_size", "csa_output_project", "csa_output_project_workspace_size",
    "csa_forward_noalloc", "csa_noalloc_scratch_bytes", "csa_index_scores_grouped", "csa_index_topk_grouped",
    "OP_COMPRESS", "OP_INDEX_TOPK", "OP_ATTEND", "OP_FORWARD",
    "FMT_F32", "FMT_BF16", "FMT_E4M3", "FMT_E4M3_BF16", "FMT_MXFP4", "FMT_MXFP4_BF16", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
FMT_F32, FMT_BF16, FMT_E4M3, FMT_E4M3_BF16, FMT_MXFP4, FMT_MXFP4_BF16 = 0, 1, 2, 3, 4, 5
OP_COMPRESS, OP_INDEX_TOPK, OP_ATTEND, OP_FORWARD = 0, 1, 2, 3

EXPORTED_SYMBOLS = (
    "csa_abi_version", "csa_status_string", "csa_last_error", "csa_row_bytes",
    "csa_state_width", "csa_state_rows", "csa_workspace_size", "csa_compress",
    "csa_index_topk", "csa_attend", "csa_forward", "csa_index_scores", "csa_topk",
    "csa_topk_workspace_size", "csa_query_project", "csa_query_project_workspace_size",
    "csa_output_project", "csa_output_project_workspace_size", "csa_forward_noalloc",
    "csa_noalloc_scratch_bytes", "csa_index_scores_grouped", "csa_index_topk_grouped",
)


class CsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"csa status {status}: {message}")
        self.status = status


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("d", "c", "rope_dim", "n_h", "c_I", "n_hI", "m",
                                              "dual", "top_k", "n_win")] + [
        ("scale", ctypes.c_float), ("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float),
        ("act_fmt", ctypes.c_int32), ("kv_fmt", ctypes.c_int32), ("idx_fmt", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("w_kv", ctypes.c_void_p), ("w_idx", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("bias_idx", ctypes.c_void_p), ("gamma_kv", ctypes.c_void_p)]


class _ProjWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_dq", "w_uq", "w_iuq", "w_w", "w_og", "w_o")] + [
        (n, ctypes.c_int32) for n in ("d_c", "g", "d_g")]


class _Cache(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("cap", ctypes.c_int32), ("win_cap", ctypes.c_int32),
                ("kv", ctypes.c_void_p), ("ki", ctypes.c_void_p), ("n_entries", ctypes.c_void_p),
                ("win", ctypes.c_void_p), ("win_pos", ctypes.c_void_p), ("state", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
                ("page_tokens", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


ABI_VERSION = 2   # the csa.h version these structures follow


_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, "libcsa.so")


def load():
    """Load libcsa.so (built in-tree by ``long_context_attention_11_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m long_context_attention_11_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    dims_p = ctypes.POINTER(_Dims)
    lib.csa_abi_version.restype = ctypes.c_int
    if lib.csa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} was built from csa.h version {lib.csa_abi_version()}, "
                           f"the binding expects {ABI_VERSION}: rebuild it")
    lib.csa_status_string.restype = ctypes.c_char_p
    lib.csa_status_string.argtypes = [ctypes.c_int]
    lib.csa_last_error.restype = ctypes.c_char_p
    lib.csa_row_bytes.restype = SZ
    lib.csa_row_bytes.argtypes = [dims_p]
    lib.csa_state_width.restype = I32
    lib.csa_state_width.argtypes = [dims_p]
    lib.csa_state_rows.restype = I32
    lib.csa_state_rows.argtypes = [dims_p]
    lib.csa_workspace_size.restype = ctypes.c_int
    lib.csa_workspace_size.argtypes = [dims_p, I32, I32, I32, I32, I32, I32, ctypes.POINTER(SZ)]
    lib.csa_compress.restype = ctypes.c_int
    lib.csa_compress.argtypes = [dims_p, ctypes.POINTER(_Weights), ctypes.POINTER(_Cache), P, I32, P, P, SZ, P]
    lib.csa_index_topk.restype = ctypes.c_int
    lib.csa_index_topk.argtypes = [dims_p, ctypes.POINTER(_Cache), P, P, P, P, I32, P, P, P, SZ, P]
    lib.csa_index_topk_grouped.restype = ctypes.c_int
    lib.csa_index_topk_grouped.argtypes = [dims_p, ctypes.POINTER(_Cache), P, P, P, P, I32, P, P, P, SZ, P]
    lib.csa_index_scores.restype = ctypes.c_int
    lib.csa_index_scores.argtypes = [dims_p, ctypes.POINTER(_Cache), P, P, P, P, I32, P, ctypes.c_int64, P]
    lib.csa_index_scores_grouped.restype = ctypes.c_int
    lib.csa_index_scores_grouped.argtypes = [dims_p, ctypes.POINTER(_Cache), P, P, P, P, I32, P, ctypes.c_int64, P]
    lib.csa_topk.restype = ctypes.c_int
    lib.csa_topk.argtypes = [dims_p, ctypes.POINTER(_Cache), P, P, I32, P, ctypes.c_int64, P, P, SZ, P]
    lib.csa_topk_workspace_size.restype = SZ
    lib.csa_topk_workspace_size.argtypes = [dims_p, I32, I32]
    lib.csa_attend.restype = ctypes.c_int
    lib.csa_attend.argtypes = [dims_p, ctypes.POINTER(_Cache), P, P, P, P, P, I32, P, P, P, SZ, P]
    lib.csa_forward.restype = ctypes.c_int
    lib.csa_forward.argtypes = [dims_p, ctypes.POINTER(_Weights), ctypes.POINTER(_Cache), P, I32, P,
                                P, P, P, P, P, P, P, P, SZ, P]
    lib.csa_forward_noalloc.restype = ctypes.c_int
    lib.csa_forward_noalloc.argtypes = [dims_p, ctypes.POINTER(_Weights), ctypes.POINTER(_Cache), P, I32, P,
                                        P, P, P, P, P, P, P, P]
    lib.csa_noalloc_scratch_bytes.restype = SZ
    lib.csa_noalloc_scratch_bytes.argtypes = []
    pw_p = ctypes.POINTER(_ProjWeights)
    lib.csa_query_project_workspace_size.restype = SZ
    lib.csa_query_project_workspace_size.argtypes = [dims_p, pw_p, I32]
    lib.csa_query_project.restype = ctypes.c_int
    lib.csa_query_project.argtypes = [dims_p, pw_p, P, I32, P, P, P, P, SZ, P]
    lib.csa_output_project_workspace_size.restype = SZ
    lib.csa_output_project_workspace_size.argtypes = [dims_p, pw_p, I32]
    lib.csa_output_project.restype = ctypes.c_int
    lib.csa_output_project.argtypes = [dims_p, pw_p, P, I32, P, P, SZ, P]
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise CsaError(status, load().csa_last_error().decode(errors="replace"))


# ----------------------------------------------------------------------------- structures

_FMT = {"f32": FMT_F32, "bf16": FMT_BF16, "e4m3": FMT_E4M3, "q": FMT_E4M3_BF16, "mxfp4": FMT_MXFP4,
        "q4": FMT_MXFP4_BF16}


@dataclass
class Dims:
    """Layer shape and formats (mirrors csa_dims).  ``kv_fmt``: "f32", "q" (E4M3 + bf16
    RoPE dims) or "q4" (MXFP4 + bf16 RoPE dims); ``idx_fmt``: "f32", "e4m3" or "mxfp4";
    ``act``: "f32" or "bf16".  dual = False with top_k > 0 is a CSA2 layer."""
    d: int
    c: int
    rope_dim: int
    n_h: int
    c_I: int
    n_hI: int
    m: int
    dual: bool
    top_k: int
    n_win: int
    act: str = "f32"
    kv_fmt: str = "f32"
    idx_fmt: str = "f32"
    scale: float = 0.0
    rope_base: float = 10000.0
    eps: float = 1e-6

    @classmethod
    def from_config(cls, cfg: dict, **over) -> "Dims":
        keys = ("d", "c", "rope_dim", "n_h", "c_I", "n_hI", "m", "dual", "top_k", "n_win", "act",
                "kv_fmt", "idx_fmt", "rope_base", "eps")
        kw = {k: cfg[k] for k in keys if k in cfg}
        kw.update(over)
        return cls(**kw)

    def struct(self) -> _Dims:
        return _Dims(self.d, self.c, self.rope_dim, self.n_h, self.c_I, self.n_hI, self.m,
                     int(bool(self.dual)), self.top_k, self.n_win, self.scale, self.rope_base,
                     self.eps, _FMT[self.act], _FMT[self.kv_fmt], _FMT[self.idx_fmt])


def _ptr(t) -> int:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def csa_abi_version() -> int:
    return load().csa_abi_version()


def csa_row_bytes(dims: Dims) -> int:
    return load().csa_row_bytes(ctypes.byref(dims.struct()))


def csa_state_width(dims: Dims) -> int:
    return load().csa_state_width(ctypes.byref(dims.struct()))


def csa_state_rows(dims: Dims) -> int:
    return load().csa_state_rows(ctypes.byref(dims.struct()))


def csa_workspace_size(dims: Dims, op: int, B: int = 1, T: int = 1, Q: int = 1, cap: int = 1,
                       q_chunk: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(load().csa_workspace_size(ctypes.byref(dims.struct()), op, B, T, Q, cap, q_chunk,
                                     ctypes.byref(out)))
    return out.value


class Cache:
    """Caller-owned cache tensors for ``B`` sequences (see csa_cache in csa.h).

    Contiguous by default: ``kv`` [B][cap][row_bytes], ``ki`` per sequence.  With
    ``block_table`` ([B][max_blocks] int32 on the device) the cache is paged: ``kv`` and ``ki``
    are pools of ``n_pages`` pages of ``page_tokens / m`` entries each (``kv``
    [n_pages][E][row_bytes]; ``ki`` [n_pages][E][c_I] bytes, or for MXFP4 per page E rows of
    element bytes then E rows of scale codes), and logical page j of sequence b is pool page
    ``block_table[b][j]``.  The window ring, its positions, the projection state and the entry
    counts stay per sequence."""

    def __init__(self, dims: Dims, B: int, cap: int, win_cap: int, device="cuda",
                 block_table=None, page_tokens: int = 128, n_pages: int = 0):
        import torch
        self.dims, self.B, self.cap, self.win_cap = dims, B, cap, win_cap
        rb = csa_row_bytes(dims)
        if rb == 0:
            raise CsaError(1, load().csa_last_error().decode())
        self.row_bytes = rb
        u8 = dict(dtype=torch.uint8, device=device)
        self.block_table = block_table
        if block_table is not None:
            if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
                raise ValueError("block_table must be an int32 [B][max_blocks] tensor")
            self.block_table = block_table.contiguous()
            self.max_blocks, self.page_tokens, self.n_pages = block_table.shape[1], page_tokens, n_pages
            groups, rows = n_pages, page_tokens // dims.m      # pool: n_pages groups of E rows
        else:
            self.max_blocks, self.page_tokens, self.n_pages = 0, 0, 0
            groups, rows = B, cap                              # one group of cap rows per sequence
        self.kv = torch.zeros((groups, rows, rb), **u8)
        if dims.top_k > 0 and dims.idx_fmt == "mxfp4":
            # per group: rows of c_I / 2 element bytes, then rows of c_I / 32 scale codes
            self.ki = torch.zeros((groups, rows * (dims.c_I // 2 + dims.c_I // 32)), **u8)
        elif dims.top_k > 0:
            kib = dims.c_I * (4 if dims.idx_fmt == "f32" else 1)
            self.ki = torch.zeros((groups, rows, kib), **u8)
        else:
            self.ki = None
        self._rows = rows
        self.n_entries = torch.zeros(B, dtype=torch.int32, device=device)
        self.win = torch.zeros((B, win_cap, rb), **u8)
        self.win_pos = torch.full((B, win_cap), -1, dtype=torch.int32, device=device)
        self.state = torch.zeros((B, csa_state_rows(dims), csa_state_width(dims)),
                                 dtype=torch.float32, device=device)

    @property
    def ki_codes(self):
        """MXFP4 keys: the element bytes, a [groups][rows][c_I / 2] view of ki (groups are
        sequences of cap rows, or pool pages)."""
        n = self._rows * (self.dims.c_I // 2)
        return self.ki[:, :n].view(self.ki.shape[0], self._rows, self.dims.c_I // 2)

    @property
    def ki_scales(self):
        """MXFP4 keys: the block scale codes, a [groups][rows][c_I / 32] view of ki."""
        n = self._rows * (self.dims.c_I // 2)
        return self.ki[:, n:].view(self.ki.shape[0], self._rows, self.dims.c_I // 32)

    def reset(self):
        self.n_entries.zero_()
        self.win_pos.fill_(-1)
        self.state.zero_()

    def struct(self) -> _Cache:
        return _Cache(self.B, self.cap, self.win_cap, _ptr(self.kv), _ptr(self.ki),
                      _ptr(self.n_entries), _ptr(self.win), _ptr(self.win_pos), _ptr(self.state),
                      _ptr(self.block_table), self.max_blocks, self.page_tokens, self.n_pages)


class Weights:
    """Compression weights (see csa_weights in csa.h): ``w_kv`` [4|2][c][d], ``w_idx``
    [4][c_I][d] (CSA), ``bias`` [2][m][c] (CSA) or [m][c] (HCA), ``bias_idx`` [2][m][c_I],
    ``gamma_kv`` [c] or None."""

    def __init__(self, w_kv, bias, w_idx=None, bias_idx=None, gamma_kv=None):
        self.w_kv, self.bias, self.w_idx, self.bias_idx, self.gamma_kv = w_kv, bias, w_idx, bias_idx, gamma_kv

    def struct(self) -> _Weights:
        return _Weights(_ptr(self.w_kv), _ptr(self.w_idx), _ptr(self.bias), _ptr(self.bias_idx),
                        _ptr(self.gamma_kv))


def _ws(ws):
    return (_ptr(ws), ws.numel() * ws.element_size()) if ws is not None else (None, 0)


def csa_compress(dims: Dims, w: Weights, cache: Cache, H, T: int, pos0, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(load().csa_compress(ctypes.byref(dims.struct()), ctypes.byref(w.struct()),
                               ctypes.byref(cache.struct()), _ptr(H), T, _ptr(pos0), wp, wn,
                               _stream(stream)))


def _check_scores(dims: Dims, t):
    """Scores are float32, or bfloat16 with the MXFP4 indexer path."""
    if t is None:
        return
    import torch
    want = torch.bfloat16 if dims.idx_fmt == "mxfp4" else torch.float32
    if t.dtype != want:
        raise ValueError(f"scores must be {want} for idx_fmt {dims.idx_fmt!r}, got {t.dtype}")


def csa_index_topk(dims: Dims, cache: Cache, qI, w, q_seq, q_pos, Q: int, idx_out,
                   scores_out=None, ws=None, stream=None):
    _check_scores(dims, scores_out)
    wp, wn = _ws(ws)
    _check(load().csa_index_topk(ctypes.byref(dims.struct()), ctypes.byref(cache.struct()),
                                 _ptr(qI), _ptr(w), _ptr(q_seq), _ptr(q_pos), Q, _ptr(idx_out),
                                 _ptr(scores_out), wp, wn, _stream(stream)))


def csa_index_topk_grouped(dims: Dims, cache: Cache, qI, w, q_seq, q_pos, Q: int, idx_out,
                           scores_out=None, ws=None, stream=None):
    """csa_index_topk for a prefill chunk's query layout (aligned groups of 16 queries of one
    sequence)."""
    _check_scores(dims, scores_out)
    wp, wn = _ws(ws)
    _check(load().csa_index_topk_grouped(ctypes.byref(dims.struct()), ctypes.byref(cache.struct()),
                                         _ptr(qI), _ptr(w), _ptr(q_seq), _ptr(q_pos), Q, _ptr(idx_out),
                                         _ptr(scores_out), wp, wn, _stream(stream)))


def csa_index_scores(dims: Dims, cache: Cache, qI, w, q_seq, q_pos, Q: int, scores, ld: int,
                     stream=None):
    _check_scores(dims, scores)
    _check(load().csa_index_scores(ctypes.byref(dims.struct()), ctypes.byref(cache.struct()),
                                   _ptr(qI), _ptr(w), _ptr(q_seq), _ptr(q_pos), Q, _ptr(scores),
                                   ld, _stream(stream)))


def csa_index_scores_grouped(dims: Dims, cache: Cache, qI, w, q_seq, q_pos, Q: int, scores, ld: int,
                             stream=None):
    """csa_index_scores for a prefill chunk's query layout (aligned groups of 16 queries of
    one sequence)."""
    _check_scores(dims, scores)
    _check(load().csa_index_scores_grouped(ctypes.byref(dims.struct()), ctypes.byref(cache.struct()),
                                           _ptr(qI), _ptr(w), _ptr(q_seq), _ptr(q_pos), Q, _ptr(scores),
                                           ld, _stream(stream)))


def csa_topk_workspace_size(dims: Dims, Q: int, cap: int) -> int:
    return load().csa_topk_workspace_size(ctypes.byref(dims.struct()), Q, cap)


def csa_topk(dims: Dims, cache: Cache, q_seq, q_pos, Q: int, scores, ld: int, idx_out, ws=None,
             stream=None):
    _check_scores(dims, scores)
    wp, wn = _ws(ws)
    _check(load().csa_topk(ctypes.byref(dims.struct()), ctypes.byref(cache.struct()), _ptr(q_seq),
                           _ptr(q_pos), Q, _ptr(scores), ld, _ptr(idx_out), wp, wn, _stream(stream)))


def csa_attend(dims: Dims, cache: Cache, q, gamma_q, sink, q_seq, q_pos, Q: int, idx, out,
               ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(load().csa_attend(ctypes.byref(dims.struct()), ctypes.byref(cache.struct()), _ptr(q),
                             _ptr(gamma_q), _ptr(sink), _ptr(q_seq), _ptr(q_pos), Q, _ptr(idx),
                             _ptr(out), wp, wn, _stream(stream)))


def csa_forward(dims: Dims, w: Weights, cache: Cache, H, T: int, pos0, q, qI, wI, gamma_q, sink,
                out, idx_out=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(load().csa_forward(ctypes.byref(dims.struct()), ctypes.byref(w.struct()),
                              ctypes.byref(cache.struct()), _ptr(H), T, _ptr(pos0), _ptr(q),
                              _ptr(qI), _ptr(wI), _ptr(gamma_q), _ptr(sink), _ptr(out),
                              _ptr(idx_out), wp, wn, _stream(stream)))


def csa_forward_noalloc(dims: Dims, w: Weights, cache: Cache, H, T: int, pos0, q, qI, wI, gamma_q, sink,
                        out, idx_out=None, stream=None):
    """csa_forward on the library's static scratch: no workspace argument, nothing allocated."""
    _check(load().csa_forward_noalloc(ctypes.byref(dims.struct()), ctypes.byref(w.struct()),
                                      ctypes.byref(cache.struct()), _ptr(H), T, _ptr(pos0), _ptr(q),
                                      _ptr(qI), _ptr(wI), _ptr(gamma_q), _ptr(sink), _ptr(out),
                                      _ptr(idx_out), _stream(stream)))


def csa_noalloc_scratch_bytes() -> int:
    return load().csa_noalloc_scratch_bytes()


class ProjWeights:
    """Weights of the projections around the path (csa_proj_weights in csa.h), bf16, each
    matrix stored transposed: ``w_dq`` [d_c][d], ``w_uq`` [n_h c][d_c], ``w_iuq``
    [n_hI c_I][d_c], ``w_w`` [n_hI][d], ``w_og`` [g][d_g][c n_h / g], ``w_o`` [d][g d_g]."""

    def __init__(self, w_dq, w_uq, w_iuq, w_w, w_og, w_o):
        self.w_dq, self.w_uq, self.w_iuq, self.w_w, self.w_og, self.w_o = w_dq, w_uq, w_iuq, w_w, w_og, w_o
        self.d_c = int(w_dq.shape[0])
        self.g, self.d_g = int(w_og.shape[0]), int(w_og.shape[1])

    def struct(self) -> _ProjWeights:
        return _ProjWeights(_ptr(self.w_dq), _ptr(self.w_uq), _ptr(self.w_iuq), _ptr(self.w_w), _ptr(self.w_og),
                            _ptr(self.w_o), self.d_c, self.g, self.d_g)


def csa_query_project_workspace_size(dims: Dims, pw: ProjWeights, T: int) -> int:
    return load().csa_query_project_workspace_size(ctypes.byref(dims.struct()), ctypes.byref(pw.struct()), T)


def csa_query_project(dims: Dims, pw: ProjWeights, h, T: int, q, qI, w, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(load().csa_query_project(ctypes.byref(dims.struct()), ctypes.byref(pw.struct()), _ptr(h), T, _ptr(q),
                                    _ptr(qI), _ptr(w), wp, wn, _stream(stream)))


def csa_output_project_workspace_size(dims: Dims, pw: ProjWeights, T: int) -> int:
    return load().csa_output_project_workspace_size(ctypes.byref(dims.struct()), ctypes.byref(pw.struct()), T)


def csa_output_project(dims: Dims, pw: ProjWeights, o, T: int, out, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(load().csa_output_project(ctypes.byref(dims.struct()), ctypes.byref(pw.struct()), _ptr(o), T, _ptr(out),
                                     wp, wn, _stream(stream)))
