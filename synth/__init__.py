"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module draws random numbers and casts them to storage types; it holds none of the
attention method's arithmetic.  Every tensor comes from a torch.Generator seeded from
(seed, tensor id, extra ids), so any chunk can be drawn again on its own.  Both the HIP
path and the CPU oracle receive exactly the same bytes: a test draws a tensor once, hands
it to the library, and gives a host copy to the oracle.

Workload shapes follow the five layer configurations the attention path is measured on:
  c1   tiny prefill, fp32: n=256, d=256, m=4, c=64 (RoPE 16), 4 heads, indexer 2x16, k=8,
       n_win=16
  c2   Flash-shaped decode: 16 sequences x 131072 tokens (32768 entries), d=4096, 64 heads
       of 512, indexer 64x128, k=512, n_win=128, E4M3+bf16 KV
  c3   Pro-shaped decode: 4 x 1048576 tokens (262144 entries), d=7168, 128 heads, k=1024
  c4a  Flash chunked prefill: a 32768-token chunk after a 1048576-token prefix
  c4b  the same after a 262144-token prefix
  c2fp4, c4afp4, c4bfp4  c2, c4a and c4b with the indexer's keys and queries in MXFP4
  c5   HCA decode: 8 x 1048576 tokens, m'=128 (8192 entries), dense, 64 heads
  c6   CSA2 (the V4.1-Flash layer): c2's shape with the single-path fold (m=4, no bias),
       index keys projected from the entry and MXFP4 main KV rows; c6fp4 with MXFP4 indexer
       keys and queries; c1v2 the same layer kind at c1's tiny fp32 shape
Value distributions: hidden states N(0,1); projection weights N(0, 1/fan_in); positional
biases and sink logits N(0, 0.1) (second argument read as the variance); queries, indexer
queries and indexer head weights N(0,1).  Synthetic cache rows (used where a decode stage is
tested on its own) are N(0,1) per dimension, the scale of an RMS-normalised row; synthetic
indexer keys are N(0, 0.25).
"""
from __future__ import annotations

import hashlib
import math

import torch

__all__ = ["CONFIGS", "config", "generator", "randn", "mxfp4_random", "weights", "hidden", "queries",
           "synthetic_cache", "row_bytes", "proj_weights", "small_ints", "SEED"]

SEED = 0

_BASE = dict(rope_base=10000.0, eps=1e-6)
# projections around the path: d_c = 1536 (Pro's, and read as Flash's), d_g = 1024 groups
_FLASH_PROJ = dict(d_c=1536, g=8, d_g=1024)
_PRO_PROJ = dict(d_c=1536, g=16, d_g=1024)

CONFIGS = {
    "c1": dict(name="c1", B=1, prefix=0, T=256, d=256, c=64, rope_dim=16, n_h=4, c_I=16, n_hI=2,
               m=4, dual=True, top_k=8, n_win=16, kv_fmt="f32", idx_fmt="f32", act="f32",
               sink=True, **_BASE),
    "c2": dict(name="c2", B=16, prefix=131072, T=1, d=4096, c=512, rope_dim=64, n_h=64, c_I=128,
               n_hI=64, m=4, dual=True, top_k=512, n_win=128, kv_fmt="q", idx_fmt="e4m3",
               act="bf16", sink=True, **_BASE, **_FLASH_PROJ),
    # c2 with the indexer's QK path in MXFP4 (the pages' later FP4 indexer revision)
    "c2fp4": dict(name="c2fp4", B=16, prefix=131072, T=1, d=4096, c=512, rope_dim=64, n_h=64,
                  c_I=128, n_hI=64, m=4, dual=True, top_k=512, n_win=128, kv_fmt="q",
                  idx_fmt="mxfp4", act="bf16", sink=True, **_BASE, **_FLASH_PROJ),
    "c3": dict(name="c3", B=4, prefix=1048576, T=1, d=7168, c=512, rope_dim=64, n_h=128, c_I=128,
               n_hI=64, m=4, dual=True, top_k=1024, n_win=128, kv_fmt="q", idx_fmt="e4m3",
               act="bf16", sink=True, **_BASE, **_PRO_PROJ),
    "c4a": dict(name="c4a", B=1, prefix=1048576, T=32768, d=4096, c=512, rope_dim=64, n_h=64,
                c_I=128, n_hI=64, m=4, dual=True, top_k=512, n_win=128, kv_fmt="q",
                idx_fmt="e4m3", act="bf16", sink=True, **_BASE, **_FLASH_PROJ),
    "c4b": dict(name="c4b", B=1, prefix=262144, T=32768, d=4096, c=512, rope_dim=64, n_h=64,
                c_I=128, n_hI=64, m=4, dual=True, top_k=512, n_win=128, kv_fmt="q",
                idx_fmt="e4m3", act="bf16", sink=True, **_BASE, **_FLASH_PROJ),
    # c4a and c4b with the indexer's QK path in MXFP4
    "c4afp4": dict(name="c4afp4", B=1, prefix=1048576, T=32768, d=4096, c=512, rope_dim=64, n_h=64,
                   c_I=128, n_hI=64, m=4, dual=True, top_k=512, n_win=128, kv_fmt="q",
                   idx_fmt="mxfp4", act="bf16", sink=True, **_BASE, **_FLASH_PROJ),
    "c4bfp4": dict(name="c4bfp4", B=1, prefix=262144, T=32768, d=4096, c=512, rope_dim=64, n_h=64,
                   c_I=128, n_hI=64, m=4, dual=True, top_k=512, n_win=128, kv_fmt="q",
                   idx_fmt="mxfp4", act="bf16", sink=True, **_BASE, **_FLASH_PROJ),
    "c5": dict(name="c5", B=8, prefix=1048576, T=1, d=4096, c=512, rope_dim=64, n_h=64, c_I=0,
               n_hI=0, m=128, dual=False, top_k=0, n_win=128, kv_fmt="q", idx_fmt="e4m3",
               act="bf16", sink=True, **_BASE, **_FLASH_PROJ),
    # CSA2 (PaperTrace §6.4, V4.1-Flash paragraph) at the Flash decode shape
    "c6": dict(name="c6", B=16, prefix=131072, T=1, d=4096, c=512, rope_dim=64, n_h=64, c_I=128,
               n_hI=64, m=4, dual=False, top_k=512, n_win=128, kv_fmt="q4", idx_fmt="e4m3",
               act="bf16", sink=True, **_BASE, **_FLASH_PROJ),
    "c6fp4": dict(name="c6fp4", B=16, prefix=131072, T=1, d=4096, c=512, rope_dim=64, n_h=64, c_I=128,
                  n_hI=64, m=4, dual=False, top_k=512, n_win=128, kv_fmt="q4", idx_fmt="mxfp4",
                  act="bf16", sink=True, **_BASE, **_FLASH_PROJ),
    "c1v2": dict(name="c1v2", B=1, prefix=0, T=256, d=256, c=64, rope_dim=16, n_h=4, c_I=16, n_hI=2,
                 m=4, dual=False, top_k=8, n_win=16, kv_fmt="f32", idx_fmt="f32", act="f32",
                 sink=True, **_BASE),
}


def config(name: str, **over) -> dict:
    """A copy of a named configuration with fields overridden."""
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    return cfg


def row_bytes(cfg: dict) -> int:
    """Bytes of one stored KV row: 4c for fp32, (c - r) E4M3 + r bf16 for "q", and for "q4"
    r bf16 + (c - r) / 2 element bytes + (c - r) / 32 scale codes padded to 128 bytes."""
    c, r = cfg["c"], cfg["rope_dim"]
    if cfg["kv_fmt"] == "f32":
        return 4 * c
    if cfg["kv_fmt"] == "q4":
        return -(-(2 * r + (c - r) // 2 + (c - r) // 32) // 128) * 128
    return c - r + 2 * r


def _seed_of(*ids) -> int:
    h = hashlib.sha256(repr(tuple(ids)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def generator(device, *ids) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed_of(*ids))
    return g


def randn(shape, std, device, *ids) -> torch.Tensor:
    """float32 N(0, std^2) drawn from a generator seeded by ``ids``."""
    g = generator(device, *ids)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def mxfp4_random(rows: int, n: int, device, *ids, lo: int = 100, hi: int = 140, mag_max: int = 7):
    """Random MXFP4 rows (n elements each): uniformly drawn element bytes [rows][n / 2] (two
    E2M1 codes each) and block scale codes [rows][n / 32] uniform in lo .. hi (by default
    2^-27 .. 2^13, so the blocks of one row often lie many octaves apart).  One block in 16
    is all zeros with scale code 127 (what an all-zero block gets), and in one row in 8 the
    last block's code is pulled 12 octaves below the row's first (clamped at lo).  Drawn
    directly as codes, so both sides decode the same bytes and no encoding is involved.
    ``mag_max`` < 7 caps each element's magnitude code (E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4,
    6 have codes 0 .. 7), keeping the sign uniform."""
    g = generator(device, *ids)
    nb = n // 32
    if mag_max >= 7:
        codes = torch.randint(0, 256, (rows, n // 2), generator=g, device=device, dtype=torch.int32)
    else:
        mag = torch.randint(0, mag_max + 1, (rows, n), generator=g, device=device, dtype=torch.int32)
        sign = torch.randint(0, 2, (rows, n), generator=g, device=device, dtype=torch.int32)
        nib = (sign << 3) | mag
        codes = nib[:, 0::2] | (nib[:, 1::2] << 4)
    scales = torch.randint(lo, hi + 1, (rows, nb), generator=g, device=device, dtype=torch.int32)
    zero = torch.rand((rows, nb), generator=g, device=device) < 1.0 / 16
    far = torch.rand((rows,), generator=g, device=device) < 1.0 / 8
    scales[:, -1] = torch.where(far, (scales[:, 0] - 12).clamp(min=lo), scales[:, -1])
    scales = torch.where(zero, torch.full_like(scales, 127), scales)
    codes = codes.view(rows, nb, 16).masked_fill(zero.unsqueeze(-1), 0).view(rows, n // 2)
    return codes.to(torch.uint8), scales.to(torch.uint8)


def _store(x: torch.Tensor, kind: str) -> torch.Tensor:
    if kind == "f32":
        return x.to(torch.float32)
    if kind == "bf16":
        return x.to(torch.bfloat16)
    if kind == "e4m3":
        return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    raise ValueError(kind)


def weights(cfg: dict, seed: int = SEED, device="cpu") -> dict:
    """Projection weights (rows = output features, [width][d]), biases, gamma and sink.

    CSA: kv_a kv_b z_a z_b [c][d]; ki_a ki_b zi_a zi_b [c_I][d]; B_a B_b [m][c];
         BI_a BI_b [m][c_I].  HCA: kv z [c][d]; B [m][c].  CSA2: kv z [c][d]; B None (no
         bias); w_ik [c_I][c] (N(0, 1/c)), the projection of the normalised entry.
    Weights are stored in the activation type (fp32 or bf16); biases, gamma (ones) and the
    sink are fp32.
    """
    d, c, cI, m = cfg["d"], cfg["c"], cfg["c_I"], cfg["m"]
    act = cfg["act"]
    std_w = 1.0 / math.sqrt(d)
    std_b = math.sqrt(0.1)
    W = {}
    names = ("kv_a", "kv_b", "z_a", "z_b") if cfg["dual"] else ("kv", "z")
    for i, nm in enumerate(names):
        W[nm] = _store(randn((c, d), std_w, device, seed, "w", nm), act)
    if cfg["dual"]:
        for nm in ("ki_a", "ki_b", "zi_a", "zi_b"):
            W[nm] = _store(randn((cI, d), std_w, device, seed, "w", nm), act)
        W["B_a"] = randn((m, c), std_b, device, seed, "b", "a")
        W["B_b"] = randn((m, c), std_b, device, seed, "b", "b")
        W["BI_a"] = randn((m, cI), std_b, device, seed, "b", "ia")
        W["BI_b"] = randn((m, cI), std_b, device, seed, "b", "ib")
    elif cfg["top_k"] > 0:
        W["B"] = None
        W["w_ik"] = _store(randn((cI, c), 1.0 / math.sqrt(c), device, seed, "w", "ik"), act)
    else:
        W["B"] = randn((m, c), std_b, device, seed, "b", "hca")
    W["gamma_kv"] = torch.ones(c, device=device, dtype=torch.float32)
    W["gamma_q"] = torch.ones(c, device=device, dtype=torch.float32)
    W["sink"] = (randn((cfg["n_h"],), std_b, device, seed, "sink") if cfg.get("sink", True)
                 else None)
    return W


def hidden(cfg: dict, seq: int, t0: int, t1: int, seed: int = SEED, device="cpu",
           chunk: int = 4096) -> torch.Tensor:
    """Hidden states of tokens t0..t1-1 of sequence ``seq``, [t1-t0][d] in the activation type.
    Drawn in aligned chunks of ``chunk`` tokens so that any range can be drawn again."""
    d = cfg["d"]
    parts = []
    c0 = (t0 // chunk) * chunk
    while c0 < t1:
        blk = randn((chunk, d), 1.0, device, seed, "h", seq, c0)
        lo, hi = max(t0, c0) - c0, min(t1, c0 + chunk) - c0
        parts.append(_store(blk[lo:hi], cfg["act"]))
        c0 += chunk
    return torch.cat(parts, 0)


def queries(cfg: dict, Q: int, seed: int = SEED, device="cpu", tag="q", mx_codes=(100, 140)) -> dict:
    """Per-query inputs: q [Q][n_h][c] (activation type), qI [Q][n_hI][c_I] (index format),
    w [Q][n_hI] (activation type).  All N(0,1), except MXFP4 q^I: random codes
    (mxfp4_random, scale codes in the range ``mx_codes``; (125, 127) is the range the MX
    scale rule gives blocks of N(0,1) values), laid out per query as element bytes then scale
    codes."""
    out = {"q": _store(randn((Q, cfg["n_h"], cfg["c"]), 1.0, device, seed, tag, "q"), cfg["act"])}
    idx = cfg["top_k"] > 0
    if idx and cfg["idx_fmt"] == "mxfp4":
        # per query: n_hI rows of element bytes, then n_hI rows of scale codes
        codes, scales = mxfp4_random(Q * cfg["n_hI"], cfg["c_I"], device, seed, tag, "qI4",
                                     lo=mx_codes[0], hi=mx_codes[1])
        out["qI"] = torch.cat([codes.view(Q, -1), scales.view(Q, -1)], dim=1).contiguous()
    elif idx:
        out["qI"] = _store(randn((Q, cfg["n_hI"], cfg["c_I"]), 1.0, device, seed, tag, "qI"),
                           cfg["idx_fmt"])
    if idx:
        out["w"] = _store(randn((Q, cfg["n_hI"]), 1.0, device, seed, tag, "w"), cfg["act"])
    return out


def synthetic_cache(cfg: dict, B: int, N: int, R: int, seed: int = SEED, device="cpu") -> dict:
    """A synthetic compressed cache for testing the decode stages on their own.

    kv  [B][N][row] uint8 rows (N(0,1) per dimension, stored in the KV format)
    ki  [B][N][c_I] indexer keys (N(0, 0.25), stored in the index format)
    win [B][R][row] window ring rows, N(0,1) like kv.
    """
    c, r = cfg["c"], cfg["rope_dim"]

    def rows(n, *ids):
        x = randn((B, n, c), 1.0, device, seed, *ids)
        if cfg["kv_fmt"] == "f32":
            return x.contiguous().view(torch.uint8).reshape(B, n, 4 * c)
        if cfg["kv_fmt"] == "q4":
            # the library's MXFP4_BF16 row: bf16 RoPE dims, element bytes, scale codes, zero
            # pad.  Drawn as codes: scale codes 125 .. 127 (the ones the MX rule gives blocks of
            # N(0,1) values) and element magnitudes up to 3 (code 5), so that rows have about
            # the RMS (1) and the range of an RMS-normalised row
            rope = x[..., c - r:].to(torch.bfloat16).contiguous().view(torch.uint8)
            el, sc = mxfp4_random(B * n, c - r, device, seed, *ids, "q4", lo=125, hi=127, mag_max=5)
            pad = torch.zeros((B, n, row_bytes(cfg) - rope.shape[-1] - el.shape[-1] - sc.shape[-1]),
                              dtype=torch.uint8, device=device)
            return torch.cat([rope, el.view(B, n, -1), sc.view(B, n, -1), pad], dim=-1).contiguous()
        nope = _store(x[..., : c - r], "e4m3")
        rope = x[..., c - r:].to(torch.bfloat16).contiguous().view(torch.uint8)
        return torch.cat([nope, rope], dim=-1).contiguous()

    out = {"kv": rows(N, "ckv"), "win": rows(R, "cwin")}
    if cfg["top_k"] > 0 and cfg["idx_fmt"] == "mxfp4":
        # per sequence: N rows of element bytes, then N rows of scale codes
        codes, scales = mxfp4_random(B * N, cfg["c_I"], device, seed, "cki4")
        out["ki"] = torch.cat([codes.view(B, -1), scales.view(B, -1)], dim=1).contiguous()
    elif cfg["top_k"] > 0:
        out["ki"] = _store(randn((B, N, cfg["c_I"]), 0.5, device, seed, "cki"), cfg["idx_fmt"])
    return out


def small_ints(shape, lo: int, hi: int, scale: float, device, *ids) -> torch.Tensor:
    """float32 tensor of integers uniform in lo..hi times ``scale`` (a power of two), drawn
    from a generator seeded by ``ids``: inputs whose sums of products stay exact in float32."""
    g = generator(device, *ids)
    return torch.randint(lo, hi + 1, shape, generator=g, device=device).to(torch.float32) * scale


def proj_weights(cfg: dict, d_c: int, g: int, d_g: int, seed: int = SEED, device="cpu",
                 exact_first: bool = False) -> dict:
    """Weights of the projections around the path, bf16, each stored transposed ([out][in]):
    w_dq [d_c][d], w_uq [n_h c][d_c], w_iuq [n_hI c_I][d_c], w_w [n_hI][d],
    w_og [g][d_g][n_h c / g], w_o [d][g d_g]; N(0, 1/fan_in).  With ``exact_first`` the maps
    applied first to their input (w_dq, w_w, w_og) take values k/64, k uniform in -2..2, so
    that with small-integer inputs their float32 sums are exact."""
    d, nq, nqI, nI = cfg["d"], cfg["n_h"] * cfg["c"], cfg["n_hI"] * cfg["c_I"], cfg["n_hI"]
    G = nq // g
    shapes = {"w_dq": (d_c, d), "w_uq": (nq, d_c), "w_iuq": (nqI, d_c), "w_w": (nI, d),
              "w_og": (g, d_g, G), "w_o": (d, g * d_g)}
    fan_in = {"w_dq": d, "w_uq": d_c, "w_iuq": d_c, "w_w": d, "w_og": G, "w_o": g * d_g}
    out = {}
    for i, (name, shp) in enumerate(shapes.items()):
        if exact_first and name in ("w_dq", "w_w", "w_og"):
            t = small_ints(shp, -2, 2, 1.0 / 64, device, seed, 700 + i)
        else:
            t = randn(shp, fan_in[name] ** -0.5, device, seed, 700 + i)
        out[name] = t.to(torch.bfloat16)
    return out
