"""Shared test helpers: marshal synthetic inputs to the HIP library and to the oracle, and
compare results under the parity rules.

Parity rules (what "matches the oracle" means):
  * top-k index sets equal, except that an index in the symmetric difference must be tied with
    the k-th largest oracle score within a relative gap of 1e-6;
  * float32 outputs within 1e-5 max abs;
  * bf16/E4M3 outputs within 2e-2 max abs and 1e-2 mean relative (sum|d| / sum|ref|);
  * stored E4M3/bf16 values: the correct rounding of some value within 2^-16 x max(|x|, row
    RMS) of the oracle's pre-storage value x (both sides decide from float32; their float32
    values differ by accumulation order, with errors on the scale of the row, e.g. where a
    rotation cancels terms).
"""
from __future__ import annotations

import numpy as np
import torch

import long_context_attention_11_amd as L
from oracle import codecs
from oracle import csa_ref as R

TOPK_TIE_REL = 1e-6
F32_MAX_ABS = 1e-5
Q_MAX_ABS = 2e-2
Q_MEAN_REL = 1e-2


def oracle_dims(cfg: dict, **over) -> R.Dims:
    kw = dict(d=cfg["d"], c=cfg["c"], rope_dim=cfg["rope_dim"], n_h=cfg["n_h"], c_I=cfg["c_I"],
              n_hI=cfg["n_hI"], m=cfg["m"], dual=cfg["dual"], top_k=cfg["top_k"],
              n_win=cfg["n_win"], kv_fmt=cfg["kv_fmt"], idx_fmt=cfg["idx_fmt"],
              rope_base=cfg["rope_base"], eps=cfg["eps"])
    kw.update(over)
    return R.Dims(**kw)


def lib_weights(W: dict, dual: bool) -> L.Weights:
    """Pack synthetic weights (synth.weights) into the ABI layout (CSA2: no bias, w_idx the
    entry-to-key projection)."""
    if dual:
        w_kv = torch.stack([W["kv_a"], W["kv_b"], W["z_a"], W["z_b"]]).contiguous()
        w_idx = torch.stack([W["ki_a"], W["ki_b"], W["zi_a"], W["zi_b"]]).contiguous()
        bias = torch.stack([W["B_a"], W["B_b"]]).contiguous()
        bias_idx = torch.stack([W["BI_a"], W["BI_b"]]).contiguous()
        return L.Weights(w_kv, bias, w_idx, bias_idx, W["gamma_kv"])
    w_kv = torch.stack([W["kv"], W["z"]]).contiguous()
    if W.get("w_ik") is not None:
        return L.Weights(w_kv, None, W["w_ik"].contiguous(), None, W["gamma_kv"])
    return L.Weights(w_kv, W["B"].contiguous(), None, None, W["gamma_kv"])


def host64(t) -> np.ndarray:
    """Exact float64 host copy of a float32/bf16 tensor."""
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def oracle_weights(W: dict) -> dict:
    out = {}
    for k, v in W.items():
        if k in ("gamma_q", "sink"):
            continue
        out[k] = None if v is None else host64(v)
    return out


def decode_rows(rows_u8: np.ndarray, cfg: dict) -> np.ndarray:
    """Stored KV rows (bytes) -> float64 values, by the oracle's codecs."""
    c, r = cfg["c"], cfg["rope_dim"]
    rows_u8 = np.ascontiguousarray(rows_u8)
    if cfg["kv_fmt"] == "f32":
        return rows_u8.view(np.float32).astype(np.float64)
    if cfg["kv_fmt"] == "q4":
        # the library's MXFP4_BF16 row: r bf16 RoPE dims, (c - r) / 2 element bytes, scales
        ne, ns = (c - r) // 2, (c - r) // 32
        rope = codecs.bf16_decode(rows_u8[..., : 2 * r].copy().view("<u2"))
        nope = codecs.mxfp4_decode(rows_u8[..., 2 * r: 2 * r + ne], rows_u8[..., 2 * r + ne: 2 * r + ne + ns])
        return np.concatenate([nope, rope], axis=-1)
    nope = codecs.e4m3_decode(rows_u8[..., : c - r])
    rope = codecs.bf16_decode(rows_u8[..., c - r:].copy().view("<u2"))
    return np.concatenate([nope, rope], axis=-1)


def decode_keys(k: torch.Tensor, cfg: dict) -> np.ndarray:
    a = k.cpu().numpy()
    if cfg["idx_fmt"] == "f32":
        return np.ascontiguousarray(a).view(np.float32).astype(np.float64)
    return codecs.e4m3_decode(a)


def keys_of(cache, b: int, lo: int, hi: int, cfg: dict) -> np.ndarray:
    """Stored indexer keys lo .. hi - 1 of sequence b, decoded by the oracle's codecs."""
    if cfg["idx_fmt"] == "mxfp4":
        return codecs.mxfp4_decode(cache.ki_codes[b, lo:hi].cpu().numpy(), cache.ki_scales[b, lo:hi].cpu().numpy())
    return decode_keys(cache.ki[b, lo:hi], cfg)


def qI_host(qI: torch.Tensor, cfg: dict) -> np.ndarray:
    if cfg["idx_fmt"] == "f32":
        return host64(qI)
    if cfg["idx_fmt"] == "mxfp4":
        a = qI.cpu().numpy()
        Q, nh, cI = a.shape[0], cfg["n_hI"], cfg["c_I"]
        codes = a[:, : nh * cI // 2].reshape(Q, nh, cI // 2)
        scales = a[:, nh * cI // 2:].reshape(Q, nh, cI // 32)
        return codecs.mxfp4_decode(codes, scales)
    return codecs.e4m3_decode(qI.cpu().numpy())


def check_topk(gpu_idx: np.ndarray, scores: np.ndarray, k: int, what: str = "") -> bool:
    """Check one query's selection against the oracle's scores.  Returns True when the sets
    are identical, False when they differ only by allowed ties (raises otherwise)."""
    V = scores.shape[0]
    g = gpu_idx[gpu_idx >= 0]
    assert np.all(gpu_idx[len(g):] == -1), f"{what}: -1 padding must trail"
    assert np.all(np.diff(g) > 0), f"{what}: indices must be strictly increasing"
    assert len(g) == 0 or (g[0] >= 0 and g[-1] < V), f"{what}: index out of the visible range"
    ref = R.topk(scores, k)
    assert len(g) == len(ref), f"{what}: selected {len(g)} entries, oracle {len(ref)}"
    diff = np.setxor1d(g, ref)
    if len(diff) == 0:
        return True
    sk = scores[ref].min()
    for s in diff:
        gap = abs(scores[s] - sk)
        assert gap <= TOPK_TIE_REL * max(abs(scores[s]), abs(sk)), (
            f"{what}: entry {s} (score {scores[s]!r}) differs from the oracle's set; "
            f"k-th score {sk!r}, relative gap {gap / max(abs(sk), 1e-300):.3g}")
    return False


# The MXFP4 indexer's stated bound: its BF16 score is the exact score rounded once unless the
# exact score lies within this many times sum_h |w_h| sum_u |q_hu k_u| of a rounding midpoint
# (dots are exact; the float64 head sum and the float64 sum of block terms where the block
# scales span many octaves round at most a few dozen times, each by 2^-53 of that sum).
BF16_SCORE_BAND = 2.0 ** -44


def check_bf16_scores(got: np.ndarray, qI: np.ndarray, w: np.ndarray, KI: np.ndarray, what: str = ""):
    """BF16 index scores of the MXFP4 path ([V]) against the oracle's exact ones for one query.
    Every score must equal the oracle's, except where the exact score lies within the stated
    band of a midpoint between two bfloat16 values; there either neighbour is accepted.
    Returns the scores the selection is checked against: the oracle's, with any such
    legitimately different GPU value in its place."""
    ref = R.bf16_index_scores(qI, w, KI)
    bad = np.flatnonzero(got != ref)
    if len(bad) == 0:
        return ref
    s = R.index_scores(qI, w, KI[bad])
    mag = (np.abs(KI[bad]) @ np.abs(qI).T) @ np.abs(w)
    band = (BF16_SCORE_BAND + 2.0 ** -40) * mag   # plus the float64 evaluation of s itself
    lo, hi = codecs.bf16_round_nearest(s - band), codecs.bf16_round_nearest(s + band)
    ok = (lo != hi) & ((got[bad] == lo) | (got[bad] == hi))
    assert ok.all(), (f"{what}: {int((~ok).sum())} bf16 scores differ from the exact score's rounding "
                      f"outside the stated band; first at {bad[~ok][:3]}: {got[bad[~ok][:3]]} vs {ref[bad[~ok][:3]]}")
    out = ref.copy()
    out[bad] = got[bad]
    return out


def assert_close_q(got: np.ndarray, ref: np.ndarray, what: str = ""):
    d = np.abs(got - ref)
    mx = d.max()
    mr = d.sum() / max(np.abs(ref).sum(), 1e-300)
    assert mx <= Q_MAX_ABS and mr <= Q_MEAN_REL, f"{what}: max abs {mx:.3g}, mean rel {mr:.3g}"
    return mx, mr


def assert_close_f32(got: np.ndarray, ref: np.ndarray, what: str = ""):
    mx = np.abs(got - ref).max()
    assert mx <= F32_MAX_ABS, f"{what}: max abs {mx:.3g}"
    return mx


def check_stored_mxfp4(codes: np.ndarray, scales: np.ndarray, ref_pre: np.ndarray, what: str = "",
                       rel: float = 2.0 ** -16):
    """Stored MXFP4 keys (element bytes [rows][n/2], scale codes [rows][n/32]) vs the oracle's
    pre-storage float64 keys [rows][n], with the tolerance of check_stored_codes: each block's
    scale must be the one the MX rule gives for a block maximum within eps of the oracle's,
    and each element, under the stored scale, the rounding of a value within eps of the
    oracle's.  Returns how many elements differ from the oracle's own encoding."""
    x = np.asarray(ref_pre, np.float64)
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) * np.ones_like(x)
    eps = rel * np.maximum(np.abs(x), rms)
    e_got = scales.astype(np.int64) - 127
    blk = lambda a: a.reshape(a.shape[:-1] + (a.shape[-1] // 32, 32))
    amax, emax = np.abs(blk(x)).max(-1), blk(eps).max(-1)
    e_lo = codecs.mxfp4_scale_exponent(np.repeat(np.maximum(amax - emax, 0.0), 32, -1))
    e_hi = codecs.mxfp4_scale_exponent(np.repeat(amax + emax, 32, -1))
    ok_s = (e_got >= e_lo) & (e_got <= e_hi)
    assert ok_s.all(), f"{what}: {int((~ok_s).sum())} block scales off the MX rule; got {e_got[~ok_s][:4]}, want {e_lo[~ok_s][:4]}"
    e_el = np.repeat(e_got, 32, -1)
    got = codecs.mxfp4_decode(codes, scales)
    rnd = lambda v: codecs.e2m1_decode(codecs.e2m1_encode_scaled(v, e_el)) * np.ldexp(1.0, e_el)
    lo, hi = rnd(x - eps), rnd(x + eps)
    ok = (got >= lo) & (got <= hi)
    assert ok.all(), (f"{what}: {int((~ok).sum())} stored elements outside the rounding of the oracle's "
                      f"value +- eps; first: got {got[~ok][:3]}, pre {x[~ok][:3]}")
    c_ref, s_ref = codecs.mxfp4_encode(x)
    return int((codecs.mxfp4_decode(codecs.mxfp4_pack(c_ref), s_ref) != got).sum())


def check_stored_codes(got_vals: np.ndarray, ref_pre: np.ndarray, fmt: str, what: str = "",
                       rel: float = 2.0 ** -16):
    """Stored values from the GPU vs the oracle's pre-storage float64 values ref_pre [rows][cols].

    Both sides compute the pre-storage value in floating point and round it to the format;
    their pre-storage values may differ by eps = rel * max(|x|, RMS of x's row) (float32
    accumulation order; rotations that cancel terms carry errors on the scale of the row).
    So the GPU's stored value must be the correct rounding of some value within eps of the
    oracle's x: round(x - eps) <= got <= round(x + eps).  Returns how many stored values
    differ from round(x)."""
    x = np.asarray(ref_pre, np.float64)
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) * np.ones_like(x)
    eps = rel * np.maximum(np.abs(x), rms)
    if fmt == "f32":
        ok = np.abs(got_vals - x) <= eps + 1e-30
        assert ok.all(), f"{what}: worst {np.max(np.abs(got_vals - x) / np.maximum(eps, 1e-30)):.3g} x tolerance"
        return 0
    if fmt == "e4m3":
        rnd = lambda v: codecs.e4m3_decode(codecs.e4m3_encode(v))
    else:
        rnd = lambda v: codecs.bf16_decode(codecs.bf16_encode(v))
    lo, hi, mid = rnd(x - eps), rnd(x + eps), rnd(x)
    ok = (got_vals >= lo) & (got_vals <= hi)
    assert ok.all(), (f"{what}: {int((~ok).sum())} stored values outside the rounding of the oracle's "
                      f"value +- eps; first: got {got_vals[~ok][:3]}, oracle {mid[~ok][:3]}, pre {x[~ok][:3]}")
    return int((got_vals != mid).sum())


def check_rounded(got_vals: np.ndarray, ref_pre: np.ndarray, bound: np.ndarray, rnd, what: str = "",
                  max_flip_frac: float = 0.02) -> int:
    """Stored values vs the oracle's pre-storage values: each stored value must be the
    rounding (``rnd``, monotone) of some value within ``bound`` of the oracle's, i.e.
    rnd(x - bound) <= got <= rnd(x + bound), and at most ``max_flip_frac`` of them may differ
    from rnd(x).  Returns how many differ."""
    x = np.asarray(ref_pre, np.float64)
    b = np.asarray(bound, np.float64) * np.ones_like(x)
    lo, hi, mid = rnd(x - b), rnd(x + b), rnd(x)
    ok = (got_vals >= lo) & (got_vals <= hi)
    assert ok.all(), (f"{what}: {int((~ok).sum())} of {ok.size} values outside the rounding of the oracle's "
                      f"value +- bound; first: got {got_vals[~ok][:3]}, oracle {mid[~ok][:3]}")
    flips = int((got_vals != mid).sum())
    assert flips <= max_flip_frac * max(1, got_vals.size), f"{what}: {flips} of {got_vals.size} differ from the rounding"
    return flips


def sum_bound(a: np.ndarray, bT: np.ndarray, ksplit_max: int = 64) -> np.ndarray:
    """Worst-case error of a float32 sum of the K products a[r, k] * bT[n, k] in any order
    (MFMA accumulation plus split-K additions): (K + ksplit) 2^-24 sum_k |a b|."""
    K = a.shape[-1]
    return (K + ksplit_max) * 2.0 ** -24 * (np.abs(a) @ np.abs(bT).T)
