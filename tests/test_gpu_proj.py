"""GPU parity of the projections around the path (csa_query_project, csa_output_project)
against the oracle (oracle/layer_ref.py), through the C ABI.

Inputs come from ``synth``.  In the exact-latent cases the first map of each side has small
integer inputs and weights k/64, so its float32 sums are exact and both sides round the same
value to bf16; the second map's float32 sums then differ from the oracle's float64 ones by
at most (K + ksplit) 2^-24 sum|a b| (``sum_bound``), and each stored value must be the
rounding of a value within that bound of the oracle's.  The realistic cases (N(0,1) inputs
and weights everywhere) are held to the output bar of the attention outputs.
"""
import numpy as np
import pytest
import torch

import long_context_attention_11_amd as L
import synth
from helpers import check_rounded, check_stored_mxfp4, host64, qI_host, sum_bound
from oracle import codecs
from oracle import layer_ref as LR
from oracle.csa_ref import Dims as ODims

pytestmark = pytest.mark.gpu
DEV = "cuda"

bf16 = lambda v: codecs.bf16_decode(codecs.bf16_encode(v))
e4m3 = lambda v: codecs.e4m3_decode(codecs.e4m3_encode(v))


def _ws(n):
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=DEV)


def _cfg(name, **over):
    cfg = synth.config(name, **over)
    return cfg


def _odims(cfg):
    return ODims(d=cfg["d"], c=cfg["c"], rope_dim=cfg["rope_dim"], n_h=cfg["n_h"], c_I=cfg["c_I"],
                 n_hI=cfg["n_hI"], m=cfg["m"], dual=cfg["dual"], top_k=cfg["top_k"], n_win=cfg["n_win"],
                 kv_fmt=cfg["kv_fmt"], idx_fmt=cfg["idx_fmt"])


def _qI_buffer(cfg, T):
    if cfg["idx_fmt"] == "mxfp4":
        return torch.zeros((T, cfg["n_hI"] * (cfg["c_I"] // 2 + cfg["c_I"] // 32)), dtype=torch.uint8, device=DEV)
    return torch.zeros((T, cfg["n_hI"], cfg["c_I"]), dtype=torch.uint8, device=DEV)


def _run_query(cfg, W, h):
    dims = L.Dims.from_config(cfg)
    pw = L.ProjWeights(**W)
    T = h.shape[0]
    q = torch.zeros((T, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device=DEV)
    qI = _qI_buffer(cfg, T)
    w = torch.zeros((T, cfg["n_hI"]), dtype=torch.bfloat16, device=DEV)
    ws = _ws(L.csa_query_project_workspace_size(dims, pw, T))
    L.csa_query_project(dims, pw, h, T, q, qI, w, ws)
    torch.cuda.synchronize()
    return q, qI, w


def _run_output(cfg, W, o):
    dims = L.Dims.from_config(cfg)
    pw = L.ProjWeights(**W)
    T = o.shape[0]
    out = torch.zeros((T, cfg["d"]), dtype=torch.bfloat16, device=DEV)
    ws = _ws(L.csa_output_project_workspace_size(dims, pw, T))
    L.csa_output_project(dims, pw, o, T, out, ws)
    torch.cuda.synchronize()
    return out


def _oracle_w(W):
    return {"dq": host64(W["w_dq"]), "uq": host64(W["w_uq"]), "iuq": host64(W["w_iuq"]), "w": host64(W["w_w"]),
            "og": host64(W["w_og"]), "o": host64(W["w_o"])}


def _check_query_exact(cfg, W, h, rows, what):
    """Exact-latent query side on the given rows: q, w and q^I against the oracle."""
    q, qI, w = _run_query(cfg, W, h)
    OW = _oracle_w(W)
    ri = torch.as_tensor(rows, device=DEV)
    hn = host64(h[ri])
    r = LR.query_projections(hn, OW, _odims(cfg))
    # the latent is exact on both sides: its float32 sum is an exact multiple of 2^-6
    assert np.all(np.abs(hn @ OW["dq"].T) < 2.0 ** 17)
    T = len(rows)
    # w = h W^w: exact before rounding on both sides
    np.testing.assert_array_equal(host64(w[ri]), r["w"], err_msg=f"{what}: w")
    b_q = sum_bound(r["cQ"], OW["uq"])
    check_rounded(host64(q[ri]).reshape(T, -1), r["q_pre"].reshape(T, -1), b_q, bf16, f"{what}: q")
    b_qI = sum_bound(r["cQ"], OW["iuq"]).reshape(T, cfg["n_hI"], cfg["c_I"])
    if cfg["idx_fmt"] == "mxfp4":
        a = qI[ri].cpu().numpy()
        nh, cI = cfg["n_hI"], cfg["c_I"]
        codes = a[:, : nh * cI // 2].reshape(T * nh, cI // 2)
        scales = a[:, nh * cI // 2:].reshape(T * nh, cI // 32)
        pre = r["qI_pre"].reshape(T * nh, cI)
        rms = np.sqrt(np.mean(pre * pre, axis=-1, keepdims=True))
        rel = float(np.max(b_qI.reshape(T * nh, cI) / np.maximum(np.abs(pre), rms)))
        check_stored_mxfp4(codes, scales, pre, f"{what}: qI", rel=max(rel, 2.0 ** -30))
    else:
        got = qI_host(qI[ri], cfg)
        check_rounded(got, r["qI_pre"], b_qI, e4m3, f"{what}: qI")


def _check_output_exact(cfg, W, o, rows, what):
    out = _run_output(cfg, W, o)
    OW = _oracle_w(W)
    ri = torch.as_tensor(rows, device=DEV)
    on = host64(o[ri]).reshape(len(rows), -1)
    r = LR.grouped_output_projection(on, OW, W["w_og"].shape[0])
    assert np.all(np.abs(r["mid_pre"]) < 2.0 ** 17)
    b = sum_bound(r["mid"], OW["o"])
    check_rounded(host64(out[ri]), r["out_pre"], b, bf16, f"{what}: out")


def _small(idx_fmt):
    # quantized-path widths (c = 512) with small d, d_c, g, d_g; n_h = 16 heads in 4 groups
    return _cfg("c2", d=256, n_h=16, n_hI=16, idx_fmt=idx_fmt)


@pytest.mark.parametrize("idx_fmt", ["e4m3", "mxfp4"])
def test_query_project_small_exact(idx_fmt):
    """37 tokens (ragged against the 64-row tiles), d = 256, d_c = 192, 16 + 16 heads."""
    cfg = _small(idx_fmt)
    W = synth.proj_weights(cfg, 192, 4, 128, seed=51, device=DEV, exact_first=True)
    h = synth.small_ints((37, cfg["d"]), -1, 1, 1.0, DEV, 51, 1).to(torch.bfloat16)
    _check_query_exact(cfg, W, h, np.arange(37), f"small {idx_fmt}")


def test_output_project_small_exact():
    """37 tokens, 16 heads of 512 in g = 4 groups projected to d_g = 128, then to d = 256."""
    cfg = _small("e4m3")
    W = synth.proj_weights(cfg, 192, 4, 128, seed=52, device=DEV, exact_first=True)
    o = synth.small_ints((37, cfg["n_h"], cfg["c"]), -1, 1, 1.0, DEV, 52, 1).to(torch.bfloat16)
    _check_output_exact(cfg, W, o, np.arange(37), "small")


@pytest.mark.parametrize("idx_fmt", ["e4m3", "mxfp4"])
def test_projections_flash_decode_exact(idx_fmt):
    """Flash shapes (d = 4096, d_c = 1536, 64 + 64 heads, g = 8, d_g = 1024) for a decode batch
    of 16 tokens: the short inputs run with split K and summed partials."""
    cfg = _cfg("c2", idx_fmt=idx_fmt)
    W = synth.proj_weights(cfg, 1536, 8, 1024, seed=53, device=DEV, exact_first=True)
    h = synth.small_ints((16, cfg["d"]), -1, 1, 1.0, DEV, 53, 1).to(torch.bfloat16)
    _check_query_exact(cfg, W, h, np.arange(16), f"flash decode {idx_fmt}")
    o = synth.small_ints((16, cfg["n_h"], cfg["c"]), -1, 1, 1.0, DEV, 53, 2).to(torch.bfloat16)
    _check_output_exact(cfg, W, o, np.arange(16), "flash decode")


def test_projections_pro_prefill_sampled():
    """Pro shapes (d = 7168, d_c = 1536, 128 heads, g = 16, d_g = 1024) for 8232 tokens: two
    row passes of the host loop (8192 + 40), sampled rows of both checked."""
    cfg = _cfg("c3")
    W = synth.proj_weights(cfg, 1536, 16, 1024, seed=54, device=DEV, exact_first=True)
    T = 8232
    rows = np.array([0, 1, 63, 64, 4097, 8191, 8192, 8200, 8231])
    h = synth.small_ints((T, cfg["d"]), -1, 1, 1.0, DEV, 54, 1).to(torch.bfloat16)
    _check_query_exact(cfg, W, h, rows, "pro prefill")
    del h
    o = synth.small_ints((T, cfg["n_h"], cfg["c"]), -1, 1, 1.0, DEV, 54, 2).to(torch.bfloat16)
    _check_output_exact(cfg, W, o, rows, "pro prefill")


def test_projections_flash_long_ragged():
    """Flash shapes for 4100 tokens: the 256x256-tile kernel of long inputs with a ragged last
    row tile (4 rows), sampled rows across its row tiles, wave rows and the tail."""
    cfg = _cfg("c2")
    W = synth.proj_weights(cfg, 1536, 8, 1024, seed=57, device=DEV, exact_first=True)
    T = 4100
    rows = np.array([0, 1, 127, 128, 255, 256, 2047, 4095, 4096, 4099])
    h = synth.small_ints((T, cfg["d"]), -1, 1, 1.0, DEV, 57, 1).to(torch.bfloat16)
    _check_query_exact(cfg, W, h, rows, "flash long")
    del h
    o = synth.small_ints((T, cfg["n_h"], cfg["c"]), -1, 1, 1.0, DEV, 57, 2).to(torch.bfloat16)
    _check_output_exact(cfg, W, o, rows, "flash long")


def test_projections_realistic_values():
    """N(0,1) hidden states and attention outputs, N(0, 1/fan_in) weights everywhere (Flash,
    300 tokens: the 128-row tiles with a ragged tail): the rounding of the latent and of the
    group outputs may differ from the oracle's at midpoints, so the outputs are held to the
    bf16 output bar."""
    cfg = _cfg("c2")
    W = synth.proj_weights(cfg, 1536, 8, 1024, seed=55, device=DEV)
    T = 300
    h = synth.randn((T, cfg["d"]), 1.0, DEV, 55, 1).to(torch.bfloat16)
    q, qI, w = _run_query(cfg, W, h)
    OW = _oracle_w(W)
    r = LR.query_projections(host64(h), OW, _odims(cfg))
    for name, got, ref in (("q", host64(q).reshape(T, -1), r["q"].reshape(T, -1)), ("w", host64(w), r["w"])):
        err = np.abs(got - ref)
        assert err.max() <= 2e-2 * max(1.0, np.abs(ref).max()), f"{name}: max abs {err.max():.3g}"
        assert err.sum() / np.abs(ref).sum() <= 1e-2, f"{name}: mean rel {err.sum() / np.abs(ref).sum():.3g}"
    o = synth.randn((T, cfg["n_h"], cfg["c"]), 1.0, DEV, 55, 2).to(torch.bfloat16)
    out = _run_output(cfg, W, o)
    ro = LR.grouped_output_projection(host64(o).reshape(T, -1), OW, 8)
    err = np.abs(host64(out) - ro["out"])
    assert err.sum() / np.abs(ro["out"]).sum() <= 1e-2, f"out: mean rel {err.sum() / np.abs(ro['out']).sum():.3g}"
    assert err.max() <= 2e-2 * max(1.0, np.abs(ro["out"]).max()), f"out: max abs {err.max():.3g}"


def test_projections_hca_and_single_token():
    """HCA layers (dual = 0) have no indexer: only q is produced (q^I and w pointers NULL).
    One token (T = 1) through both sides at Flash shapes."""
    cfg = _cfg("c5")
    dims = L.Dims.from_config(cfg)
    W = synth.proj_weights(cfg, 1536, 8, 1024, seed=56, device=DEV, exact_first=True)
    pw = L.ProjWeights(W["w_dq"], W["w_uq"], None, None, W["w_og"], W["w_o"])
    h = synth.small_ints((1, cfg["d"]), -1, 1, 1.0, DEV, 56, 1).to(torch.bfloat16)
    q = torch.zeros((1, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device=DEV)
    ws = _ws(L.csa_query_project_workspace_size(dims, pw, 1))
    L.csa_query_project(dims, pw, h, 1, q, None, None, ws)
    torch.cuda.synchronize()
    OW = _oracle_w(W)
    hn = host64(h)
    cQ = LR.to_bf16(hn @ OW["dq"].T)
    q_pre = cQ @ OW["uq"].T
    check_rounded(host64(q).reshape(1, -1), q_pre, sum_bound(cQ, OW["uq"]), bf16, "hca q")
    o = synth.small_ints((1, cfg["n_h"], cfg["c"]), -1, 1, 1.0, DEV, 56, 2).to(torch.bfloat16)
    _check_output_exact(cfg, W, o, np.arange(1), "single token")
