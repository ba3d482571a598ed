"""Shared test helpers: marshal synthetic inputs to the HIP library and to the oracle, and
compare results under the parity rules.

Parity rules (what "matches the oracle" means):
  * top-k index sets equal, except that an index in the symmetric difference must be tied with
    the k-th largest oracle score within a relative gap of 1e-6;
  * float32 outputs within 1e-5 max abs;
  * bf16/E4M3 outputs within 2e-2 max abs and 1e-2 mean relative (sum|d| / sum|ref|);
  * stored E4M3/bf16 codes equal, or one code apart where the oracle's value lies within
    2^-16 of the rounding midpoint between them, relative to the larger of the value and its
    row's RMS (both sides decide from float32; their float32 values differ by accumulation
    order, with errors on the scale of the row, e.g. where a rotation cancels terms).
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
    """Pack synthetic weights (synth.weights) into the ABI layout."""
    if dual:
        w_kv = torch.stack([W["kv_a"], W["kv_b"], W["z_a"], W["z_b"]]).contiguous()
        w_idx = torch.stack([W["ki_a"], W["ki_b"], W["zi_a"], W["zi_b"]]).contiguous()
        bias = torch.stack([W["B_a"], W["B_b"]]).contiguous()
        bias_idx = torch.stack([W["BI_a"], W["BI_b"]]).contiguous()
        return L.Weights(w_kv, bias, w_idx, bias_idx, W["gamma_kv"])
    w_kv = torch.stack([W["kv"], W["z"]]).contiguous()
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
    nope = codecs.e4m3_decode(rows_u8[..., : c - r])
    rope = codecs.bf16_decode(rows_u8[..., c - r:].copy().view("<u2"))
    return np.concatenate([nope, rope], axis=-1)


def decode_keys(k: torch.Tensor, cfg: dict) -> np.ndarray:
    a = k.cpu().numpy()
    if cfg["idx_fmt"] == "f32":
        return np.ascontiguousarray(a).view(np.float32).astype(np.float64)
    return codecs.e4m3_decode(a)


def qI_host(qI: torch.Tensor, cfg: dict) -> np.ndarray:
    if cfg["idx_fmt"] == "f32":
        return host64(qI)
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


def _neighbours_e4m3(code: np.ndarray):
    v = codecs.e4m3_decode(code)
    return v


def check_stored_codes(got_vals: np.ndarray, ref_pre: np.ndarray, fmt: str, what: str = ""):
    """Stored values from the GPU vs the oracle's pre-storage float64 values.

    The oracle rounds ref_pre (via float32) to the format.  Where the GPU's code differs, it
    must be the other neighbour of a rounding midpoint that ref_pre sits next to (within
    2^-16 of max(|value|, row RMS)), i.e. a decision the two float32 values may legitimately
    take differently.  ref_pre is [rows][cols].  Returns the number of such flips."""
    ref_pre = np.asarray(ref_pre, np.float64)
    row_rms = np.sqrt(np.mean(ref_pre * ref_pre, axis=-1, keepdims=True)) * np.ones_like(ref_pre)
    if fmt == "f32":
        assert np.abs(got_vals - ref_pre).max() <= 1e-5 * max(1.0, np.abs(ref_pre).max()), what
        return 0
    if fmt == "e4m3":
        ref_vals = codecs.e4m3_decode(codecs.e4m3_encode(ref_pre))
    else:
        ref_vals = codecs.bf16_decode(codecs.bf16_encode(ref_pre))
    bad = np.nonzero(got_vals != ref_vals)
    if len(bad[0]) == 0:
        return 0
    g, r, x, rms = got_vals[bad], ref_vals[bad], ref_pre[bad], row_rms[bad]
    mid = 0.5 * (g + r)
    near = np.abs(x - mid) <= 2.0 ** -16 * np.maximum(np.abs(x), rms)
    # the two codes must be adjacent: no representable value strictly between them
    if fmt == "e4m3":
        allv = np.unique(codecs.e4m3_values()[~np.isnan(codecs.e4m3_values())])
        lo, hi = np.minimum(g, r), np.maximum(g, r)
        between = np.searchsorted(allv, hi, "left") - np.searchsorted(allv, lo, "right")
        adjacent = between == 0
    else:
        adjacent = np.abs(g - r) <= 2.0 ** -7 * np.maximum(np.abs(g), np.abs(r))
    ok = near & adjacent
    assert ok.all(), (f"{what}: {int((~ok).sum())} stored values differ beyond a midpoint flip; "
                      f"first: got {g[~ok][:3]}, oracle {r[~ok][:3]}, pre {x[~ok][:3]}")
    return int(ok.sum())
