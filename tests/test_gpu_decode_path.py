"""GPU parity of the decode step the benchmark times: ``csa_forward`` with one new token per
sequence at the full Flash (16 x 32768 entries, k = 512) and Pro (4 x 262144 entries,
k = 1024) shapes, so that more entries are visible than top-k keeps and the selection runs
through the fused launches (threshold pass + one-token projection, final pass + fold).

Four consecutive positions 4 N0 .. 4 N0 + 3 run per sequence; the last one completes entry N0.
The cache holds N0 synthetic entries, their keys and a window ring of synthetic rows for the
128 positions before 4 N0; the projection state ring holds the projections of the 8 tokens
before 4 N0, computed by the oracle from those tokens' hidden states (so both sides know
them exactly, as float32).  Per step every query's selection (tie rule), its BF16 scores with
MXFP4 keys (stated band) and its output are checked; afterwards the window rows of the four
new tokens and the new entry and key are checked against the oracle's fold of the same hidden
states.
"""
import numpy as np
import pytest
import torch

import long_context_attention_11_amd as L
import synth
from helpers import (assert_close_q, check_bf16_scores, check_stored_codes, check_stored_mxfp4,
                     check_topk, decode_rows, host64, keys_of, lib_weights, oracle_dims, oracle_weights,
                     qI_host)
from oracle import codecs
from oracle import csa_ref as R
from paging import logical, paged_cache, store_logical

pytestmark = pytest.mark.gpu
DEV = "cuda"
PATHS = ("kv_a", "kv_b", "z_a", "z_b", "ki_a", "ki_b", "zi_a", "zi_b")


def _i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def _mx_encode_rows(x: np.ndarray):
    """float64 rows [n][c_I] -> (element bytes [n][c_I/2], scale codes [n][c_I/32]) by the
    oracle's MX encoder (inputs handed to the library; nothing flows back into the oracle)."""
    c, s = codecs.mxfp4_encode(x)
    return codecs.mxfp4_pack(c), s


def _decode_path(name, idx_fmt="e4m3", realistic_mx=False, seed=51, paged=False):
    cfg = synth.config(name, idx_fmt=idx_fmt)
    dims = L.Dims.from_config(cfg)
    od = oracle_dims(cfg)
    B, m, k, nw = cfg["B"], cfg["m"], cfg["top_k"], cfg["n_win"]
    N = cfg["prefix"] // m          # capacity: the bench's
    N0 = N - 8                      # complete entries before the steps
    tau0 = m * N0
    steps = m
    print(f"decode path {name} idx={idx_fmt} realistic_mx={realistic_mx} paged={paged}: B={B} N0={N0} k={k}",
          flush=True)

    cache = paged_cache(dims, B, N, nw, seed=seed) if paged else L.Cache(dims, B=B, cap=N, win_cap=nw)
    sc = synth.synthetic_cache(cfg, B, N, nw, seed=seed, device=DEV)
    cache.win.copy_(sc["win"])
    if idx_fmt == "mxfp4" and realistic_mx:
        # keys as the MX rule encodes N(0, 0.25) values (scale codes near those a fold gives)
        kx = synth.randn((B, N, cfg["c_I"]), 0.5, "cpu", seed, "ckx").numpy().astype(np.float64)
        el, scl = _mx_encode_rows(kx.reshape(B * N, -1))
        ki0 = torch.cat([torch.from_numpy(el).view(B, -1), torch.from_numpy(scl).view(B, -1)], 1)
    else:
        ki0 = sc["ki"].view(torch.uint8)
    store_logical(cache, kv=sc["kv"], ki=ki0)
    pool = cache
    cache = logical(pool)
    cache.n_entries.fill_(N0)
    wp = np.full((B, nw), -1, dtype=np.int32)
    for j in range(tau0 - nw, tau0):
        wp[:, j % nw] = j
    cache.win_pos.copy_(torch.from_numpy(wp))

    W = synth.weights(cfg, seed=seed, device=DEV)
    OW = oracle_weights(W)
    # hidden states of the 8 tokens before the steps and of the steps' tokens
    Hs = torch.stack([synth.hidden(cfg, b, tau0 - 2 * m, tau0 + steps, seed=seed, device=DEV) for b in range(B)])
    Hn = [host64(Hs[b]) for b in range(B)]
    Pn = [{p: R.project(Hn[b], OW[p]) for p in PATHS} for b in range(B)]   # [2m + steps][width]
    # projection state ring: token j in slot j % 2m, columns in the order of PATHS, float32
    state = np.zeros((B, 2 * m, L.csa_state_width(dims)), np.float32)
    for b in range(B):
        row = np.concatenate([Pn[b][p] for p in PATHS], axis=1).astype(np.float32)
        for r in range(2 * m):
            state[b, (tau0 - 2 * m + r) % (2 * m)] = row[r]
    cache.state.copy_(torch.from_numpy(state))
    state64 = state.astype(np.float64)

    # the queries of every step; MXFP4 q^I either random codes over a wide scale range or the
    # MX rule's encoding of N(0,1) values
    qs = synth.queries(cfg, B * steps, seed=seed, device=DEV, tag="path")
    if idx_fmt == "mxfp4" and realistic_mx:
        qx = synth.randn((B * steps * cfg["n_hI"], cfg["c_I"]), 1.0, "cpu", seed, "qx").numpy().astype(np.float64)
        el, scl = _mx_encode_rows(qx)
        Q = B * steps
        qs["qI"] = torch.cat([torch.from_numpy(el).view(Q, -1), torch.from_numpy(scl).view(Q, -1)], 1).to(DEV).contiguous()

    # inputs the oracle reads, taken before the steps overwrite any of them
    ki_all = [keys_of(cache, b, 0, N0, cfg) for b in range(B)]
    ring0 = [decode_rows(cache.win[b].cpu().numpy(), cfg) for b in range(B)]
    kv_u8 = cache.kv.cpu().numpy()

    lw = lib_weights(W, True)
    ws = torch.empty(L.csa_workspace_size(dims, L.OP_FORWARD, B=B, T=1, cap=N), dtype=torch.uint8, device=DEV)
    outs, idxs = [], []
    for t in range(steps):
        rows = [b * steps + t for b in range(B)]
        out = torch.zeros((B, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device=DEV)
        idx = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
        L.csa_forward(dims, lw, pool, Hs[:, 2 * m + t:2 * m + t + 1].contiguous(), 1, _i32([tau0 + t] * B),
                      qs["q"][rows].contiguous(), qs["qI"][rows].contiguous(), qs["w"][rows].contiguous(),
                      W["gamma_q"], W["sink"], out, idx, ws)
        outs.append(out)
        idxs.append(idx)
    torch.cuda.synchronize()
    print(f"decode path {name}: {steps} steps ran, checking", flush=True)
    cache = logical(pool)

    q, qI, w = host64(qs["q"]), qI_host(qs["qI"], cfg), host64(qs["w"])
    sink = host64(W["sink"])
    c, r = cfg["c"], cfg["rope_dim"]
    assert np.all(cache.n_entries.cpu().numpy() == N0 + 1), "the fourth step completes entry N0"
    for b in range(B):
        # the new tokens' window rows: the a-path row finalized at its own position
        new_pos = tau0 + np.arange(steps)
        raw_fin = R.finalize_kv(Pn[b]["kv_a"][2 * m:], new_pos, OW["gamma_kv"], od)
        raw_new, _ = R.store_kv(raw_fin, od)
        g_raw = decode_rows(cache.win[b, new_pos % nw].cpu().numpy(), cfg)
        assert np.array_equal(cache.win_pos[b, new_pos % nw].cpu().numpy(), new_pos)
        check_stored_codes(g_raw[:, :c - r], raw_fin[:, :c - r], "e4m3", f"{name} seq {b} window/nope")
        check_stored_codes(g_raw[:, c - r:], raw_fin[:, c - r:], "bf16", f"{name} seq {b} window/rope")

        # entry N0: a rows of the four new tokens, b rows of the four before (seeded state)
        prev = {p: state64[b, [(tau0 - m + i) % (2 * m) for i in range(m)], off:off + wd]
                for p, off, wd in _state_columns(cfg)}
        cur = {p: Pn[b][p][2 * m:] for p in PATHS}
        pre = R.csa_fold(cur["kv_a"], cur["kv_b"], cur["z_a"], cur["z_b"], OW["B_a"], OW["B_b"], m,
                         prev_b=(prev["kv_b"], prev["z_b"]))
        kpre = R.csa_fold(cur["ki_a"], cur["ki_b"], cur["zi_a"], cur["zi_b"], OW["BI_a"], OW["BI_b"], m,
                          prev_b=(prev["ki_b"], prev["zi_b"]))
        fin = R.finalize_kv(pre, np.array([m * N0]), OW["gamma_kv"], od)
        g_ent = decode_rows(cache.kv[b, N0:N0 + 1].cpu().numpy(), cfg)
        check_stored_codes(g_ent[:, :c - r], fin[:, :c - r], "e4m3", f"{name} seq {b} new entry/nope")
        check_stored_codes(g_ent[:, c - r:], fin[:, c - r:], "bf16", f"{name} seq {b} new entry/rope")
        if idx_fmt == "mxfp4":
            check_stored_mxfp4(cache.ki_codes[b, N0:N0 + 1].cpu().numpy(), cache.ki_scales[b, N0:N0 + 1].cpu().numpy(),
                               kpre, f"{name} seq {b} new key")
        else:
            check_stored_codes(keys_of(cache, b, N0, N0 + 1, cfg), kpre, "e4m3", f"{name} seq {b} new key")

        # every step's query: V = N0 > k visible entries (the new entry is never visible)
        for t in range(steps):
            i = b * steps + t
            tau = tau0 + t
            V = R.visible_entries(tau, m, N0)
            assert V == N0 > k
            sc = R.scores_for_topk(qI[i], w[i], ki_all[b][:V], od)
            gi = idxs[t][b].cpu().numpy()
            what = f"{name} seq {b} tau={tau}"
            same = check_topk(gi, sc, k, what)
            sel = R.topk(sc, k) if same else gi[gi >= 0]
            wpos = R.window_positions(tau, nw)
            old = wpos < tau0
            win_rows = np.empty((len(wpos), c))
            win_rows[old] = ring0[b][wpos[old] % nw]
            win_rows[~old] = raw_new[wpos[~old] - tau0]
            keys = np.concatenate([decode_rows(kv_u8[b, sel], cfg), win_rows])
            o_ref = R.attend(q[i], tau, keys, None, sink, od)
            assert_close_q(host64(outs[t][b:b + 1])[0], o_ref, what + " out")


def _state_columns(cfg):
    c, cI = cfg["c"], cfg["c_I"]
    off, cols = 0, []
    for p in PATHS:
        wd = c if p in ("kv_a", "kv_b", "z_a", "z_b") else cI
        cols.append((p, off, wd))
        off += wd
    return cols


def test_c2_forward_decode_path_full_size():
    """Flash decode at full size through csa_forward, E4M3 indexer keys."""
    _decode_path("c2")


def test_c2_forward_decode_path_full_size_mxfp4_wide_scales():
    """The same with MXFP4 keys and queries whose block scales span up to 40 octaves (all-zero
    blocks, rows whose blocks lie 12 octaves apart): the indexer's exact per-block path."""
    _decode_path("c2", idx_fmt="mxfp4")


def test_c2_forward_decode_path_full_size_mxfp4_mx_rule_inputs():
    """MXFP4 keys and queries as the MX rule encodes N(0, 0.25) keys and N(0, 1) queries."""
    _decode_path("c2", idx_fmt="mxfp4", realistic_mx=True)


def test_c3_forward_decode_path_full_size():
    """Pro decode at full size (4 x 262144 entries, 128 heads, k = 1024) through csa_forward."""
    _decode_path("c3")


def test_c2_forward_decode_path_full_size_paged():
    """Flash decode at full size through csa_forward on a paged cache (128-token pages of 32
    entries, shuffled over the pool): the new entry and key are written through the table."""
    _decode_path("c2", paged=True)


def test_c2_forward_decode_path_full_size_mxfp4_paged():
    """The same with MXFP4 keys, wide block scales, paged."""
    _decode_path("c2", idx_fmt="mxfp4", paged=True)
