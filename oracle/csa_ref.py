"""CPU oracle of Compressed Sparse Attention (CSA) and of its dense heavily-compressed variant (HCA).

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 numpy written from the pages' definitions.
It may be imported by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``; the product path (the HIP library and its binding) never imports, links or
calls anything here, and nothing here imports the product path.

Sources (cited by tag below):
  [RN] "DeepSeekV4技术报告阅读笔记" (DeepSeek-V4 technical-report reading notes, zouxinn.github.io)
  [DD] "DeepSeek-V4 架构设计深度解析" (architecture deep dive, blog.sysu-sam.com)
  [PT] "02 · DeepSeek-V4: 压缩注意力撑起 1M 上下文" (PaperTrace analysis, yayajjiang.github.io)
  [EX] "DeepSeek V4 架构解读: CSA、HCA、mHC 与 Muon" (researchpapers.dev explainer)
  [WY] "DeepSeek-V4 技术报告分析学习" (blog.weyung.cc)

Positions are 0-based: token j sits at position j.  Where the pages leave a step open, the
reading taken is stated at the function that takes it.

Pins (what each function is checked against, in tests/test_oracle_*.py):
  fold          column sums of the softmax weights; constant rows; zero logits -> mean;
                which tokens reach which entry (the m = 4 worked example in [PT] §2.1)
  rmsnorm       output RMS is 1 for gamma = 1
  rope          a single key at position p gives the output R_{p - tau} v; shifting every
                position by the same amount leaves the output unchanged ([RN] §2.5.2)
  index_scores  one head with w = 1 reduces to ReLU(q.K); E4M3 dot products are exact
                (checked against exact rational arithmetic)
  topk          brute-force rank counting on small inputs
  attend        m = 1 with every entry selected, no sink, a window of one token and the b
                path switched off reduces to dense causal MQA (torch SDPA in float64);
                sink limits and sum of weights < 1 ([RN] §2.5.4 eq. 27)
  codecs        the E4M3 and bfloat16 formats against their bit definitions and torch casts
  CSA2          the single-path fold without bias (closed forms; no token of another block
                reaches an entry); index keys from the entry (linear in the normalised entry,
                blind to the entry's scale and position); MXFP4 main rows (worked blocks);
                m = 1 with every entry selected reduces to dense causal MQA
The learned meaning of the weights (whether trained values make a good model) cannot be
checked without trained weights: that part is parity unpinned and out of scope.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import codecs

__all__ = [
    "Dims",
    "softmax_columns",
    "project",
    "csa_fold",
    "hca_fold",
    "rmsnorm",
    "rope_rotate",
    "finalize_kv",
    "store_kv",
    "store_index_keys",
    "index_keys_from_entries",
    "compress_sequence",
    "compress_entries",
    "raw_rows",
    "visible_entries",
    "window_positions",
    "index_scores",
    "bf16_index_scores",
    "scores_for_topk",
    "topk",
    "attention_weights",
    "attend",
    "query_step",
]


@dataclass(frozen=True)
class Dims:
    """Shape and format parameters of one attention layer.

    d        hidden size of h_t                          ([RN] §2.3.1, H in R^{n x d})
    c        width of a KV entry and of a query head     ([RN] §2.3.1 and eq. 19)
    rope_dim number of trailing dimensions under RoPE     ([RN] §2.5.2: the last 64)
    n_h      query heads                                  ([RN] §2.3.3)
    c_I      indexer key / query width                    ([RN] §2.3.2)
    n_hI     indexer heads                                ([RN] §2.3.2)
    m        tokens per compressed entry (m for CSA, m' for HCA)
    dual     True: overlapping a|b compression (CSA); False: single path (HCA, [RN] §2.4,
             and CSA2)
    top_k    entries kept per query; 0 means every visible entry (HCA, [RN] eq. 26).  A
             single-path layer with top_k > 0 is CSA2 ([PT] §6.4, V4.1-Flash paragraph):
             no overlapping windows, no in-block bias, index keys projected from the entry
    n_win    sliding-window length over uncompressed tokens ([RN] §2.5.3; [PT] §2.4)
    kv_fmt   "f32", "q" (E4M3 for the non-RoPE dims, bfloat16 for the RoPE dims) or "q4"
             (MXFP4 for the non-RoPE dims, bfloat16 for the RoPE dims: CSA2's FP4 main KV)
    idx_fmt  "f32", "e4m3" or "mxfp4" (indexer keys and queries)
    """

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
    kv_fmt: str = "f32"
    idx_fmt: str = "f32"
    rope_base: float = 10000.0
    eps: float = 1e-6
    scale: float | None = None

    @property
    def softmax_scale(self) -> float:
        # Reading: the pages write the logit as q^T k ([RN] eq. 27) and explain the usual
        # 1/sqrt(d_k) scaling in general terms ([WY]); the scale taken is 1/sqrt(c).
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.c)


# --------------------------------------------------------------------------- compression


def softmax_columns(logits: np.ndarray, axis: int) -> np.ndarray:
    """Softmax taken along ``axis`` separately for every other index ([RN] eq. 11: the
    row-softmax normalises each column over the 2m stacked rows).  -inf logits get weight 0."""
    mx = np.max(logits, axis=axis, keepdims=True)
    e = np.exp(logits - mx)
    return e / np.sum(e, axis=axis, keepdims=True)


def project(H: np.ndarray, Wt: np.ndarray) -> np.ndarray:
    """C = H . W  ([RN] eqs. 9-10 and 20-21).  ``Wt`` is W transposed: [c][d], row u holds
    column u of W, so the result is H @ Wt.T with shape [n][c]."""
    return np.asarray(H, np.float64) @ np.asarray(Wt, np.float64).T


def csa_fold(Ca, Cb, Za, Zb, Ba, Bb, m: int, prev_b=None, return_weights: bool = False):
    """Overlapping dual-window compression ([RN] §2.3.1 eqs. 11-12; [PT] §2.1 worked m = 4 case).

    Ca, Cb, Za, Zb: [n][c] projections of n consecutive tokens that start at a block boundary;
    only the n // m complete blocks are folded.  Entry i (local block i) takes the a-rows of
    its own m tokens and the b-rows of the m tokens of the block before it; the 2m logits
    Z + B are soft-maxed per column and the 2m rows are summed with those weights.

    ``prev_b`` is (Cb, Zb) of the block just before local block 0, or None when local block 0
    is the first block of the sequence: then, as the reading notes state after eq. 12, its b
    logits are -inf and its b values 0, so only the a path contributes.
    Ba, Bb: [m][c] learned positional biases (reading: R^{m x c}; the notes garble the second
    dimension, but the bias is added to Z in R^{. x c} column by column).
    """
    Ca, Cb, Za, Zb = (np.asarray(x, np.float64) for x in (Ca, Cb, Za, Zb))
    n, c = Ca.shape
    nb = n // m
    la = Za[: nb * m].reshape(nb, m, c) + Ba
    va = Ca[: nb * m].reshape(nb, m, c)
    lb = np.full((nb, m, c), -np.inf)
    vb = np.zeros((nb, m, c))
    if nb > 1:
        lb[1:] = Zb[: (nb - 1) * m].reshape(nb - 1, m, c) + Bb
        vb[1:] = Cb[: (nb - 1) * m].reshape(nb - 1, m, c)
    if prev_b is not None and nb > 0:
        pCb, pZb = (np.asarray(x, np.float64) for x in prev_b)
        lb[0] = pZb + Bb
        vb[0] = pCb
    logits = np.concatenate([la, lb], axis=1)  # [nb][2m][c]
    values = np.concatenate([va, vb], axis=1)
    S = softmax_columns(logits, axis=1)
    out = np.sum(S * values, axis=1)
    return (out, S) if return_weights else out


def hca_fold(C, Z, B, m: int, return_weights: bool = False):
    """Heavily-compressed fold ([RN] §2.4.1 eqs. 22-23): each of the n // m blocks of m
    tokens is soft-maxed per column over its own m logits Z + B (B in R^{m x c}) and summed.
    Blocks do not overlap and there is no second path.

    CSA2's compression ([PT] §6.4, V4.1-Flash paragraph: eqs. 9-12 without the overlapping
    windows and the in-block positional bias) is read as this fold with m = 4 and no bias:
    pass B = None."""
    C, Z = np.asarray(C, np.float64), np.asarray(Z, np.float64)
    n, c = C.shape
    nb = n // m
    logits = Z[: nb * m].reshape(nb, m, c) + (0.0 if B is None else B)
    S = softmax_columns(logits, axis=1)
    out = np.sum(S * C[: nb * m].reshape(nb, m, c), axis=1)
    return (out, S) if return_weights else out


def rmsnorm(x, gamma, eps: float):
    """RMSNorm(x) = gamma * x / sqrt(mean(x^2) + eps) over the last axis ([DD] §3.4 gives
    x / RMS(x) * gamma with RMS = sqrt(mean(x^2)); eps is the usual guard, 1e-6 here).
    Applied to every query head and to the single KV head ([RN] §2.5.1; [PT] §2.4)."""
    x = np.asarray(x, np.float64)
    g = np.ones(x.shape[-1]) if gamma is None else np.asarray(gamma, np.float64)
    return g * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope_rotate(x, pos, rope_dim: int, base: float):
    """Rotate the last ``rope_dim`` dimensions of x by position ``pos`` ([RN] §2.5.2).

    Reading: adjacent pairs (c - r + 2j, c - r + 2j + 1), j < r/2, turn by the angle
    pos * base^(-2j/r), so that R_p^T = R_{-p} and R_p R_q = R_{p+q}.  ``pos`` broadcasts
    against x's leading axes; negative positions de-rotate.  Angles are formed in float64.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    if rope_dim == 0:
        return x
    c = x.shape[-1]
    half = rope_dim // 2
    theta = base ** (-2.0 * np.arange(half) / rope_dim)
    ang = np.asarray(pos, np.float64)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    ev = x[..., c - rope_dim :: 2].copy()
    od = x[..., c - rope_dim + 1 :: 2].copy()
    x[..., c - rope_dim :: 2] = ev * cos - od * sin
    x[..., c - rope_dim + 1 :: 2] = ev * sin + od * cos
    return x


def finalize_kv(x, pos, gamma, dims: Dims):
    """A KV row as attention sees it: RMSNorm with gamma_kv, then RoPE at its position.

    Reading: entry i sits at position m*i (the first token of its own a-block); a raw window
    row of token j sits at position j.  Norm first, rotation second."""
    return rope_rotate(rmsnorm(x, gamma, dims.eps), pos, dims.rope_dim, dims.rope_base)


def store_kv(y, dims: Dims):
    """Round finalized KV rows to their storage format.

    Returns (values, row_bytes): the float64 values attention reads back, and the bytes of
    each stored row.  "f32": c float32.  "q": c - r E4M3 bytes followed by r bfloat16
    (little-endian) — 448 + 128 = 576 bytes for c = 512, r = 64 ([EX] key-numbers table;
    [PT] §2.5).
    """
    y = np.asarray(y, np.float64)
    c, r = dims.c, dims.rope_dim
    if dims.kv_fmt == "f32":
        v = codecs.to_f32(y)
        return v, v.astype(np.float32).view(np.uint8).reshape(y.shape[:-1] + (4 * c,))
    if dims.kv_fmt == "q4":
        # CSA2's FP4 main KV ([PT] §6.4: main KV from FP8 down to FP4).  Reading: the dims
        # that were E4M3 become MXFP4 (blocks of 32 sharing an E8M0 scale, the OCP MX rule
        # as for the FP4 indexer keys); the RoPE dims stay bfloat16.  Bytes: packed element
        # codes, then the block scale codes, then the bfloat16 dims.
        codes, scales = codecs.mxfp4_encode(y[..., : c - r])
        packed = codecs.mxfp4_pack(codes)
        rope = codecs.bf16_encode(y[..., c - r :])
        vals = np.concatenate([codecs.mxfp4_decode(packed, scales), codecs.bf16_decode(rope)], axis=-1)
        rope_b = rope.astype("<u2").view(np.uint8).reshape(y.shape[:-1] + (2 * r,))
        return vals, np.concatenate([packed, scales, rope_b], axis=-1)
    nope = codecs.e4m3_encode(y[..., : c - r])
    rope = codecs.bf16_encode(y[..., c - r :])
    vals = np.concatenate([codecs.e4m3_decode(nope), codecs.bf16_decode(rope)], axis=-1)
    rope_b = rope.astype("<u2").view(np.uint8).reshape(y.shape[:-1] + (2 * r,))
    return vals, np.concatenate([nope, rope_b], axis=-1)


def store_index_keys(k, dims: Dims):
    """Round indexer keys to storage: float32, E4M3 with unit scale, or MXFP4 (the pages'
    later FP4 indexer path, [PT] §3.3).  Returns (values, bytes); for MXFP4 the
    bytes are the packed element codes followed by the block scale codes, per key."""
    k = np.asarray(k, np.float64)
    if dims.idx_fmt == "f32":
        v = codecs.to_f32(k)
        return v, v.astype(np.float32).view(np.uint8).reshape(k.shape[:-1] + (4 * k.shape[-1],))
    if dims.idx_fmt == "mxfp4":
        codes, scales = codecs.mxfp4_encode(k)
        packed = codecs.mxfp4_pack(codes)
        return codecs.mxfp4_decode(packed, scales), np.concatenate([packed, scales], axis=-1)
    code = codecs.e4m3_encode(k)
    return codecs.e4m3_decode(code), code


def index_keys_from_entries(pre, W_ik, gamma, dims: Dims):
    """CSA2's indexer keys, projected from the main KV entries ([PT] §6.4, V4.1-Flash
    paragraph: the index keys are no longer compressed on their own but projected from the
    main entry).  Reading: K^I_s = RMSNorm(C^Comp_s) . W^IK with W^IK in R^{c x c_I}, taken
    from the normalised entry before RoPE (the key then carries no position, as the V4
    indexer keys carry none) and before the entry is rounded to storage.  ``W_ik`` is
    W^IK transposed: [c_I][c]."""
    return rmsnorm(pre, gamma, dims.eps) @ np.asarray(W_ik, np.float64).T


def _paths(H, W):
    """Projections of every path listed in the weight dict W (arrays [width][d])."""
    return {name: project(H, W[name]) for name in W["paths"]}


def compress_sequence(H, W, dims: Dims):
    """Compress a whole sequence of n tokens (positions 0..n-1).

    W holds the transposed projection matrices and biases:
      CSA: "kv_a","kv_b","z_a","z_b" [c][d]; "ki_a","ki_b","zi_a","zi_b" [c_I][d];
           "B_a","B_b" [m][c]; "BI_a","BI_b" [m][c_I]; "gamma_kv" [c] or None.
      HCA: "kv","z" [c][d]; "B" [m][c]; "gamma_kv".
      CSA2 (single path, top_k > 0): "kv","z" [c][d]; "B" None (no bias); "w_ik" [c_I][c];
           "gamma_kv".
    Returns a dict with
      "entry_pre"  [n//m][c]    folded entries before RMSNorm/RoPE (float64)
      "entry_fin"  [n//m][c]    finalized entries (before rounding to storage)
      "entry"      [n//m][c]    stored values, "entry_bytes" their bytes
      "ki_pre"     [n//m][c_I]  folded indexer keys (CSA only), "ki" stored values, "ki_bytes"
      "raw_fin"/"raw"/"raw_bytes" [n][c]: window rows of every token (finalized C^a_j, or C_j
                                   for HCA, at position j).
    Reading for the indexer keys ([RN] §2.3.2: one shared K^IComp; [DD] §3.2: "the same
    compression, smaller output width"): the same overlapping fold with its own weights of
    width c_I, and no RMSNorm or RoPE, which the pages apply only to the core-attention
    query and KV heads.
    """
    H = np.asarray(H, np.float64)
    n = H.shape[0]
    m = dims.m
    nb = n // m
    out = {}
    if dims.dual:
        P = {k: project(H, W[k]) for k in ("kv_a", "kv_b", "z_a", "z_b", "ki_a", "ki_b", "zi_a", "zi_b")}
        pre = csa_fold(P["kv_a"], P["kv_b"], P["z_a"], P["z_b"], W["B_a"], W["B_b"], m)
        ki = csa_fold(P["ki_a"], P["ki_b"], P["zi_a"], P["zi_b"], W["BI_a"], W["BI_b"], m)
        raw_src = P["kv_a"]
        out["ki_pre"] = ki
        out["ki"], out["ki_bytes"] = store_index_keys(ki, dims)
    else:
        C, Z = project(H, W["kv"]), project(H, W["z"])
        pre = hca_fold(C, Z, W.get("B"), m)
        raw_src = C
        if dims.top_k > 0:
            ki = index_keys_from_entries(pre, W["w_ik"], W.get("gamma_kv"), dims)
            out["ki_pre"] = ki
            out["ki"], out["ki_bytes"] = store_index_keys(ki, dims)
    pos_e = m * np.arange(nb)
    fin = finalize_kv(pre, pos_e, W.get("gamma_kv"), dims)
    out["entry_pre"], out["entry_fin"] = pre, fin
    out["entry"], out["entry_bytes"] = store_kv(fin, dims)
    rfin = finalize_kv(raw_src, np.arange(n), W.get("gamma_kv"), dims)
    out["raw_fin"] = rfin
    out["raw"], out["raw_bytes"] = store_kv(rfin, dims)
    return out


def compress_entries(H_of, entries, W, dims: Dims):
    """Compress selected entries of a long sequence without touching the rest.

    ``H_of(j0, j1)`` returns the hidden states of tokens j0..j1-1 (float64 [j1-j0][d]).
    For entry i, CSA needs tokens m(i-1)..m(i+1)-1 (only m(i)..m(i+1)-1 for i = 0);
    HCA needs tokens m'i..m'(i+1)-1.  Returns the same per-entry keys as compress_sequence
    ("entry_pre", "entry_fin", "entry", "entry_bytes", and for CSA "ki_pre", "ki", "ki_bytes"),
    each stacked in the order of ``entries``.
    """
    m = dims.m
    rows = {k: [] for k in ("entry_pre", "ki_pre")}
    for i in entries:
        i = int(i)
        if dims.dual:
            cur = H_of(m * i, m * (i + 1))
            Pc = _paths(cur, {"paths": ("kv_a", "z_a", "ki_a", "zi_a"), **W})
            prev = None
            prevI = None
            if i > 0:
                pv = H_of(m * (i - 1), m * i)
                Pp = _paths(pv, {"paths": ("kv_b", "z_b", "ki_b", "zi_b"), **W})
                prev = (Pp["kv_b"], Pp["z_b"])
                prevI = (Pp["ki_b"], Pp["zi_b"])
            zc = np.zeros_like(Pc["kv_a"])
            zi = np.zeros_like(Pc["ki_a"])
            e = csa_fold(Pc["kv_a"], zc, Pc["z_a"], zc, W["B_a"], W["B_b"], m, prev_b=prev)
            k = csa_fold(Pc["ki_a"], zi, Pc["zi_a"], zi, W["BI_a"], W["BI_b"], m, prev_b=prevI)
            rows["entry_pre"].append(e[0])
            rows["ki_pre"].append(k[0])
        else:
            cur = H_of(m * i, m * (i + 1))
            e = hca_fold(project(cur, W["kv"]), project(cur, W["z"]), W.get("B"), m)
            rows["entry_pre"].append(e[0])
    out = {"entry_pre": np.array(rows["entry_pre"])}
    pos_e = m * np.asarray(entries, np.float64)
    out["entry_fin"] = finalize_kv(out["entry_pre"], pos_e, W.get("gamma_kv"), dims)
    out["entry"], out["entry_bytes"] = store_kv(out["entry_fin"], dims)
    if dims.dual:
        out["ki_pre"] = np.array(rows["ki_pre"])
    elif dims.top_k > 0:
        out["ki_pre"] = index_keys_from_entries(out["entry_pre"], W["w_ik"], W.get("gamma_kv"), dims)
    if "ki_pre" in out:
        out["ki"], out["ki_bytes"] = store_index_keys(out["ki_pre"], dims)
    return out


def raw_rows(H_rows, positions, W, dims: Dims):
    """Window rows of the given tokens: C^a_j (C_j for HCA) finalized at position j.

    Reading ([RN] §2.3.2 and §2.5.3 "uncompressed KV entries"; [PT] §2.4 "KV of the most
    recent n_win uncompressed tokens"): the raw KV of token j is its own a-path row, which
    adds no weights beyond the pages' and makes the m = 1 case collapse to dense attention.
    Returns (finalized, stored values, bytes)."""
    src = project(H_rows, W["kv_a"] if dims.dual else W["kv"])
    fin = finalize_kv(src, np.asarray(positions, np.float64), W.get("gamma_kv"), dims)
    vals, b = store_kv(fin, dims)
    return fin, vals, b


# --------------------------------------------------------------------------- selection


def visible_entries(tau: int, m: int, n_entries: int) -> int:
    """Number of entries a query at position tau may use: min(tau // m, n_entries).

    Reading: the block that contains tau is never used, even at its last token, because the
    pages drop the entry of the block that holds the query ([RN] §2.3.2 after eq. 17, and
    §2.5.3; [DD] §3.4; [PT] §2.4).  With 0-based positions that is s < floor(tau / m)."""
    return max(0, min(int(tau) // m, int(n_entries)))


def window_positions(tau: int, n_win: int) -> np.ndarray:
    """Positions of the sliding-window rows of a query at tau: max(0, tau-n_win+1) .. tau.
    Reading: the window includes the query's own token, so the key set is never empty."""
    return np.arange(max(0, int(tau) - n_win + 1), int(tau) + 1)


def index_scores(qI, w, KI):
    """Lightning-indexer scores I_{t,s} = sum_h w_{t,h} * ReLU(q^I_{t,h} . K^I_s)
    ([RN] §2.3.2 eq. 16; [DD] §3.2; [PT] §2.2).  qI [n_hI][c_I], w [n_hI], KI [V][c_I] -> [V].
    With E4M3 inputs every dot product here is exact in float64."""
    dots = np.asarray(KI, np.float64) @ np.asarray(qI, np.float64).T  # [V][n_hI]
    return np.maximum(dots, 0.0) @ np.asarray(w, np.float64)


def stored_scores(scores, dims: Dims):
    """The scores top-k selects from, given float64 scores: as computed, or with an MXFP4 QK
    path their rounding to the nearest bfloat16.  Exact when the float64 scores are; for the
    MXFP4 path ``scores_for_topk`` gives the rounding of the exact score in every case."""
    if dims.idx_fmt == "mxfp4":
        return codecs.bf16_round_nearest(scores)
    return np.asarray(scores, np.float64)


def _fraction_score(qI, w, k):
    """sum_h w_h ReLU(q_h . k) in exact rational arithmetic (every float is a dyadic rational)."""
    from fractions import Fraction
    total = Fraction(0)
    kf = [Fraction(float(x)) for x in k]
    for h in range(qI.shape[0]):
        dot = sum((Fraction(float(a)) * b for a, b in zip(qI[h], kf)), Fraction(0))
        if dot > 0:
            total += Fraction(float(w[h])) * dot
    return total


def _bf16_of_fraction(x) -> float:
    """The bfloat16 value nearest to the rational x, ties to the even significand."""
    from fractions import Fraction
    if x == 0:
        return 0.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    # a = f 2^e with f in [1, 2): keep 8 significant bits, round half to even
    n = round(a / Fraction(2) ** (e - 7))          # Python rounds a Fraction half to even
    v = math.ldexp(float(n), e - 7)
    return -v if x < 0 else v


def bf16_index_scores(qI, w, KI):
    """The pages' BF16 index scores of the FP4 indexer path ([PT] §3.3: with the QK path in
    FP4 the scores drop from FP32 to BF16): each exact score sum_h w_h ReLU(q_h . K_s)
    rounded once to the nearest bfloat16, ties to even.

    float64 holds the score exactly only while its terms span few enough octaves (MXFP4
    block scales can span many), so each score is first evaluated in float64 with a bound on
    that evaluation's error: a sum of n exactly representable products carries at most
    gamma_n = n u / (1 - n u) (u = 2^-53) times the sum of the terms' magnitudes, whatever the
    order, and the ReLU and the head weights add the head count to n.  When both ends of that
    interval round to the same bfloat16, so does the exact score (rounding is monotonic);
    otherwise the score is recomputed in exact rational arithmetic and rounded from there."""
    qI = np.asarray(qI, np.float64)
    w = np.asarray(w, np.float64)
    KI = np.asarray(KI, np.float64)
    s = index_scores(qI, w, KI)
    mag = (np.abs(KI) @ np.abs(qI).T) @ np.abs(w)
    n = qI.shape[-1] + qI.shape[0] + 2
    err = 2.0 * n * 2.0 ** -53 * mag
    err = err + 2.0 ** -52 * (np.abs(s) + err)   # the rounding of s -/+ err itself
    lo = codecs.bf16_round_nearest(s - err)
    hi = codecs.bf16_round_nearest(s + err)
    out = codecs.bf16_round_nearest(s)
    for j in np.flatnonzero(lo != hi):
        out[j] = _bf16_of_fraction(_fraction_score(qI, w, KI[j]))
    return out


def scores_for_topk(qI, w, KI, dims: Dims):
    """The scores top-k selects from for one query: float64 scores (exact for E4M3 and for
    float32 inputs of these sizes), or with an MXFP4 QK path the BF16 scores."""
    if dims.idx_fmt == "mxfp4":
        return bf16_index_scores(qI, w, KI)
    return index_scores(qI, w, KI)


def topk(scores, k: int) -> np.ndarray:
    """Indices of the k largest scores, as a set emitted in increasing index order
    ([RN] eq. 17).  Reading: when V <= k every entry is taken; equal scores go to the lower
    index; -0 counts as +0 (numeric comparison)."""
    scores = np.asarray(scores, np.float64)
    V = scores.shape[0]
    if V <= k:
        return np.arange(V)
    order = np.lexsort((np.arange(V), -scores))  # primary: score descending; then index
    return np.sort(order[:k])


# --------------------------------------------------------------------------- attention


def attention_weights(q_t, keys, sink, dims: Dims):
    """Per-head softmax weights with the sink in the denominator ([RN] §2.5.4 eq. 27):
    s_j = exp(z_j) / (sum_k exp(z_k) + exp(z'_h)), z_j = scale * q_t . key_j.
    q_t [n_h][c] (already normed and rotated), keys [K][c], sink [n_h] or None (no sink).
    Returns [n_h][K]."""
    z = dims.softmax_scale * (np.asarray(q_t, np.float64) @ np.asarray(keys, np.float64).T)
    mx = np.max(z, axis=1)
    if sink is not None:
        mx = np.maximum(mx, np.asarray(sink, np.float64))
    e = np.exp(z - mx[:, None])
    den = np.sum(e, axis=1)
    if sink is not None:
        den = den + np.exp(np.asarray(sink, np.float64) - mx)
    return e / den[:, None]


def attend(q, tau: int, keys, gamma_q, sink, dims: Dims):
    """Shared-KV MQA for one query token at position tau ([RN] eq. 19 / eq. 26).

    q [n_h][c] raw query heads; keys [K][c] stored KV rows (selected entries and window rows,
    K = V, shared by every head).  Each head is RMS-normalised with gamma_q and rotated to tau
    ([RN] §2.5.1-2.5.2); the output o = sum_j s_j key_j is de-rotated by -tau on the RoPE
    dims so that it carries only relative positions ([RN] §2.5.2; the report's "-i" read as
    the query position).  Returns [n_h][c]."""
    qt = rope_rotate(rmsnorm(q, gamma_q, dims.eps), tau, dims.rope_dim, dims.rope_base)
    s = attention_weights(qt, keys, sink, dims)
    o = s @ np.asarray(keys, np.float64)
    return rope_rotate(o, -tau, dims.rope_dim, dims.rope_base)


def query_step(tau: int, q, qI, w, gamma_q, sink, entries, ki, raw_of, n_entries: int, dims: Dims,
               sel=None):
    """The whole path for one query at position tau.

    entries [N][c] and ki [N][c_I] are the stored values of the sequence's compressed cache;
    ``raw_of(positions)`` returns stored window rows [len][c].  For CSA the indexer scores
    the visible entries and top-k selects; for HCA (top_k == 0) every visible entry is used
    ([RN] §2.4.2).  One softmax runs over the selected entries and the window rows together,
    with the sink (reading: [PT] §2.4 has the window rows join the compressed entries in
    attention; [DD] §3.4's "compressed output + window output" is not taken).
    ``sel`` overrides the selection (used to check a result whose selection is not unique).
    Returns (out [n_h][c], selected indices, scores or None)."""
    V = visible_entries(tau, dims.m, n_entries)
    scores = None
    if sel is None:
        if dims.top_k == 0:
            sel = np.arange(V)
        else:
            scores = scores_for_topk(qI, w, ki[:V], dims)
            sel = topk(scores, dims.top_k)
    sel = np.asarray(sel, dtype=np.int64)
    keys = np.concatenate([np.asarray(entries)[sel], raw_of(window_positions(tau, dims.n_win))], axis=0)
    return attend(q, tau, keys, gamma_q, sink, dims), sel, scores
