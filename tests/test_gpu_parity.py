"""GPU parity: the HIP library (through its C ABI) against the float64 CPU oracle.

Every input is drawn once by ``synth`` and handed to both sides; nothing the GPU computes is
fed to the oracle, except where a selection is not unique (tied scores, or a storage rounding
decision both sides may legitimately take differently): then the GPU's choice is first
checked to be a valid one and the remaining values are checked for that choice.
"""
import numpy as np
import pytest
import torch

import long_context_attention_11_amd as L
import synth
from helpers import (assert_close_f32, assert_close_q, check_bf16_scores, check_stored_codes, check_topk,
                     decode_keys, decode_rows, host64, lib_weights, oracle_dims, oracle_weights,
                     keys_of, qI_host, check_stored_mxfp4)
from oracle import codecs
from oracle import csa_ref as R
from paging import logical, paged_cache, store_logical

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def _ws(n):
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=DEV)


def _compress_chunks(dims, W, cache, Hs, chunks):
    """Feed hidden states [B][n][d] to csa_compress in the given chunk lengths."""
    lw = lib_weights(W, dims.dual)
    B = Hs.shape[0]
    p = 0
    for T in chunks:
        ws = _ws(L.csa_workspace_size(dims, L.OP_COMPRESS, B=B, T=T))
        L.csa_compress(dims, lw, cache, Hs[:, p:p + T].contiguous(), T, _i32([p] * B), ws)
        p += T
    torch.cuda.synchronize()


def _check_cache_vs_oracle(cfg, cache, b, comp, n_tokens, what):
    """Stored entries, indexer keys and window rows of sequence b vs the oracle."""
    m, c, r = cfg["m"], cfg["c"], cfg["rope_dim"]
    nb = n_tokens // m
    assert int(cache.n_entries[b]) == nb, f"{what}: n_entries"
    flips = _check_rows(cfg, cache.kv[b, :nb].cpu().numpy(), comp["entry_fin"], what + " entries")
    if cfg["top_k"] > 0:
        # CSA2's keys are a 512-term float32 projection of the entry: their pre-storage values
        # may differ from the oracle's by up to 512 x 2^-24 x sum |y| |W^IK| (about 2^-11 of the
        # key's RMS at these sizes), against the fold's 2^-16 for CSA's folded keys
        rel = 2.0 ** -16 if cfg["dual"] else 2.0 ** -11
        if cfg["idx_fmt"] == "mxfp4":
            flips += check_stored_mxfp4(cache.ki_codes[b, :nb].cpu().numpy(), cache.ki_scales[b, :nb].cpu().numpy(),
                                        comp["ki_pre"], what + " index keys", rel=rel)
        elif cfg["idx_fmt"] == "f32":
            assert_close_f32(keys_of(cache, b, 0, nb, cfg), comp["ki_pre"], what + " index keys")
        else:
            flips += check_stored_codes(keys_of(cache, b, 0, nb, cfg), comp["ki_pre"], "e4m3", what + " index keys",
                                        rel=rel)
    # window ring: the last min(win_cap, n) tokens
    wp = cache.win_pos[b].cpu().numpy()
    for j in range(max(0, n_tokens - cache.win_cap), n_tokens):
        slot = j % cache.win_cap
        assert wp[slot] == j, f"{what}: ring slot {slot} holds {wp[slot]}, want {j}"
    js = np.arange(max(0, n_tokens - cache.win_cap), n_tokens)
    flips += _check_rows(cfg, cache.win[b, js % cache.win_cap].cpu().numpy(), comp["raw_fin"][js], what + " window")
    return flips


def _check_rows(cfg, rows_u8, fin, what):
    """Stored KV rows (bytes) vs the oracle's finalized rows: float32, or each stored code the
    rounding of a value within eps of the oracle's (E4M3 or MXFP4 for the non-RoPE dims,
    bf16 for the RoPE dims).  Returns the number of codes that differ from the oracle's."""
    c, r = cfg["c"], cfg["rope_dim"]
    got = decode_rows(rows_u8, cfg)
    if cfg["kv_fmt"] == "f32":
        assert_close_f32(got, fin, what)
        return 0
    flips = check_stored_codes(got[:, c - r:], fin[:, c - r:], "bf16", what + "/rope")
    if cfg["kv_fmt"] == "q4":
        ne = (c - r) // 2
        flips += check_stored_mxfp4(rows_u8[:, 2 * r: 2 * r + ne], rows_u8[:, 2 * r + ne: 2 * r + ne + (c - r) // 32],
                                    fin[:, : c - r], what + "/nope")
    else:
        flips += check_stored_codes(got[:, : c - r], fin[:, : c - r], "e4m3", what + "/nope")
    return flips


# ----------------------------------------------------------------------------- config 1


@pytest.mark.parametrize("paged", [False, True])
def test_c1_forward_matches_oracle(paged):
    """Tiny fp32 prefill (n=256, d=256, m=4, c=64, 4 heads, k=8, n_win=16): every query.  The
    queries come from the hidden states through the low-rank query path (eqs. 13-15 and 18,
    d_c = 64), computed in float64 and handed to both sides as the same float32 arrays.
    Paged: 8-token pages (2 entries each) in a shuffled pool."""
    cfg = synth.config("c1")
    dims = L.Dims.from_config(cfg)
    od = oracle_dims(cfg)
    T, m, k = cfg["T"], cfg["m"], cfg["top_k"]
    W = synth.weights(cfg, device=DEV)
    H = synth.hidden(cfg, 0, 0, T, device=DEV)
    PW = {n: host64(t) for n, t in synth.proj_weights(cfg, 64, 1, 64, device=DEV).items()}
    hn = host64(H)
    cQ = hn @ PW["w_dq"].T                                              # eq. 13
    f32 = lambda a, shape: torch.as_tensor(a.reshape(shape), dtype=torch.float32, device=DEV).contiguous()
    qs = {"q": f32(cQ @ PW["w_uq"].T, (T, cfg["n_h"], cfg["c"])),        # eq. 18
          "qI": f32(cQ @ PW["w_iuq"].T, (T, cfg["n_hI"], cfg["c_I"])),   # eq. 14
          "w": f32(hn @ PW["w_w"].T, (T, cfg["n_hI"]))}                  # eq. 15
    cache = (paged_cache(dims, 1, T // m, T + cfg["n_win"], seed=1, page_tokens=8) if paged
             else L.Cache(dims, B=1, cap=T // m, win_cap=T + cfg["n_win"]))
    out = torch.zeros((T, cfg["n_h"], cfg["c"]), dtype=torch.float32, device=DEV)
    idx = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    ws = _ws(L.csa_workspace_size(dims, L.OP_FORWARD, B=1, T=T, cap=cache.cap))
    L.csa_forward(dims, lib_weights(W, True), cache, H.unsqueeze(0).contiguous(), T, _i32([0]),
                  qs["q"], qs["qI"], qs["w"], W["gamma_q"], W["sink"], out, idx, ws)
    torch.cuda.synchronize()

    OW = oracle_weights(W)
    comp = R.compress_sequence(host64(H), OW, od)
    _check_cache_vs_oracle(cfg, logical(cache), 0, comp, T, "c1")
    q, qI, w = host64(qs["q"]), host64(qs["qI"]), host64(qs["w"])
    sink = host64(W["sink"])
    gi, go = idx.cpu().numpy(), out.cpu().numpy().astype(np.float64)
    ties = 0
    for tau in range(T):
        o_ref, sel, sc = R.query_step(tau, q[tau], qI[tau], w[tau], None, sink, comp["entry"],
                                      comp["ki"], lambda p: comp["raw"][p], T // m, od)
        if not check_topk(gi[tau], sc, k, f"c1 tau={tau}"):
            ties += 1
            o_ref = R.query_step(tau, q[tau], qI[tau], w[tau], None, sink, comp["entry"], comp["ki"],
                                 lambda p: comp["raw"][p], T // m, od, sel=gi[tau][gi[tau] >= 0])[0]
        assert_close_f32(go[tau], o_ref, f"c1 out tau={tau}")
    assert ties <= 2


@pytest.mark.parametrize("paged", [False, True])
def test_c1_chunked_compress_equals_whole(paged):
    """Ragged chunks (not multiples of m, a single token, a block split across calls) build the
    same cache as the whole-sequence oracle: the projection state carries across calls.
    Paged: 4-token pages (one entry each)."""
    cfg = synth.config("c1")
    dims = L.Dims.from_config(cfg)
    od = oracle_dims(cfg)
    B, n = 2, 203
    W = synth.weights(cfg, seed=3, device=DEV)
    Hs = torch.stack([synth.hidden(cfg, b, 0, n, seed=3, device=DEV) for b in range(B)])
    cache = paged_cache(dims, B, 64, 32, seed=3, page_tokens=4) if paged else L.Cache(dims, B=B, cap=64, win_cap=32)
    _compress_chunks(dims, W, cache, Hs, [5, 1, 2, 50, 3, 142])
    cache = logical(cache)
    OW = oracle_weights(W)
    for b in range(B):
        comp = R.compress_sequence(host64(Hs[b]), OW, od)
        _check_cache_vs_oracle(cfg, cache, b, comp, n, f"c1 chunked seq {b}")


# ----------------------------------------------------------------------------- quantized, small


def _qcfg(**over):
    return synth.config("c2", **over)


@pytest.mark.parametrize("idx_fmt", ["e4m3", "mxfp4"])
def test_q_compress_chunked_matches_oracle(idx_fmt):
    """E4M3/bf16 storage, Flash dims (d=4096, c=512, c_I=128), indexer keys in E4M3 or MXFP4:
    2 sequences x 301 tokens in ragged chunks; stored codes match the oracle up to midpoint
    flips."""
    cfg = _qcfg(idx_fmt=idx_fmt)
    dims = L.Dims.from_config(cfg)
    od = oracle_dims(cfg)
    B, n = 2, 301
    W = synth.weights(cfg, seed=5, device=DEV)
    Hs = torch.stack([synth.hidden(cfg, b, 0, n, seed=5, device=DEV) for b in range(B)])
    cache = L.Cache(dims, B=B, cap=128, win_cap=128)
    _compress_chunks(dims, W, cache, Hs, [7, 1, 100, 64, 129])
    OW = oracle_weights(W)
    flips = 0
    for b in range(B):
        comp = R.compress_sequence(host64(Hs[b]), OW, od)
        flips += _check_cache_vs_oracle(cfg, cache, b, comp, n, f"q chunked seq {b}")
    assert flips < 50


@pytest.mark.parametrize("idx_fmt", ["e4m3", "mxfp4"])
def test_q_compress_single_token_steps(idx_fmt):
    """Decode-style compression: 17 sequences (two 16-row projection tiles, the second
    ragged) get a 3-token prefix and then 20 one-token steps, which take the step path
    (projection straight into the state ring, fold from the ring).  Every stored entry,
    indexer key and window row matches the oracle up to midpoint flips."""
    cfg = _qcfg(idx_fmt=idx_fmt)
    dims = L.Dims.from_config(cfg)
    od = oracle_dims(cfg)
    B, n = 17, 23
    W = synth.weights(cfg, seed=8, device=DEV)
    Hs = torch.stack([synth.hidden(cfg, b, 0, n, seed=8, device=DEV) for b in range(B)])
    cache = L.Cache(dims, B=B, cap=16, win_cap=128)
    _compress_chunks(dims, W, cache, Hs, [3] + [1] * (n - 3))
    OW = oracle_weights(W)
    flips = 0
    for b in range(B):
        comp = R.compress_sequence(host64(Hs[b]), OW, od)
        flips += _check_cache_vs_oracle(cfg, cache, b, comp, n, f"q single-token seq {b}")
    assert flips < 50


@pytest.mark.parametrize("paged,chunks", [(False, (100, 1, 127, 72)), (True, (100, 1, 127, 72)),
                                          (False, (127, 1, 1, 171))])
def test_hca_compress_matches_oracle(paged, chunks):
    """HCA (m'=128, single path, no indexer): 2 sequences x 300 tokens in chunks; paged: one
    entry per 128-token page.  Chunks (127, 1, 1, 171): the one-token step at position 127
    completes entry 0 (the one-token fold over all 128 rows of a block)."""
    cfg = synth.config("c5")
    dims = L.Dims.from_config(cfg)
    od = oracle_dims(cfg)
    B, n = 2, 300
    W = synth.weights(cfg, seed=6, device=DEV)
    Hs = torch.stack([synth.hidden(cfg, b, 0, n, seed=6, device=DEV) for b in range(B)])
    cache = paged_cache(dims, B, 8, 128, seed=6) if paged else L.Cache(dims, B=B, cap=8, win_cap=128)
    print(f"hca compress paged={paged} chunks={chunks}", flush=True)
    _compress_chunks(dims, W, cache, Hs, list(chunks))
    cache = logical(cache)
    OW = oracle_weights(W)
    for b in range(B):
        comp = R.compress_sequence(host64(Hs[b]), OW, od)
        _check_cache_vs_oracle(cfg, cache, b, comp, n, f"hca seq {b}")


def _synthetic_decode_setup(cfg, B, N, R_win, taus, seed=11, sink=True, n_entries=None, paged=False):
    """Synthetic cache (contiguous, or paged through a shuffled block table) + one query per
    listed (seq, tau)."""
    dims = L.Dims.from_config(cfg)
    cache = paged_cache(dims, B, N, R_win, seed=seed) if paged else L.Cache(dims, B=B, cap=N, win_cap=R_win)
    sc = synth.synthetic_cache(cfg, B, N, R_win, seed=seed, device=DEV)
    cache.win.copy_(sc["win"])
    store_logical(cache, kv=sc["kv"], ki=sc["ki"].view(torch.uint8) if cfg["top_k"] > 0 else None)
    ne = n_entries if n_entries is not None else [N] * B
    cache.n_entries.copy_(_i32(ne))
    # ring positions: the R_win tokens ending at each sequence's largest query position
    wp = np.full((B, R_win), -1, dtype=np.int32)
    for b in range(B):
        t_end = max(t for (s, t) in taus if s == b)
        for j in range(max(0, t_end - R_win + 1), t_end + 1):
            wp[b, j % R_win] = j
    cache.win_pos.copy_(torch.from_numpy(wp))
    Q = len(taus)
    qs = synth.queries(cfg, Q, seed=seed, device=DEV)
    W = {"sink": synth.randn((cfg["n_h"],), 0.1 ** 0.5, DEV, seed, "sink") if sink else None,
         "gamma_q": torch.ones(cfg["c"], device=DEV)}
    q_seq = _i32([s for s, _ in taus])
    q_pos = _i32([t for _, t in taus])
    return dims, cache, qs, W, q_seq, q_pos


def _oracle_cache(cfg, cache, b):
    entries = decode_rows(cache.kv[b].cpu().numpy(), cfg)
    ki = keys_of(cache, b, 0, cache.cap, cfg) if cfg["top_k"] > 0 else None
    win = decode_rows(cache.win[b].cpu().numpy(), cfg)
    wp = cache.win_pos[b].cpu().numpy()

    def raw_of(pos):
        # the window rows the ring actually holds (a slot holding another position is absent)
        pos = np.asarray(pos)
        slots = pos % cache.win_cap
        return win[slots[wp[slots] == pos]]
    return entries, ki, raw_of


def _run_index_attend_and_check(cfg, dims, cache, qs, W, q_seq, q_pos, taus, check_scores=True):
    Q, k = len(taus), cfg["top_k"]
    od = oracle_dims(cfg)
    idx = torch.full((Q, max(k, 1)), -7, dtype=torch.int32, device=DEV)
    sdt = torch.bfloat16 if cfg["idx_fmt"] == "mxfp4" else torch.float32
    scores = torch.zeros((Q, cache.cap), dtype=sdt, device=DEV) if check_scores else None
    out = torch.zeros((Q, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device=DEV)
    if cfg["top_k"] > 0:
        ws = _ws(L.csa_workspace_size(dims, L.OP_INDEX_TOPK, Q=Q, cap=cache.cap))
        L.csa_index_topk(dims, cache, qs["qI"], qs["w"], q_seq, q_pos, Q, idx, scores, ws)
    ws = _ws(L.csa_workspace_size(dims, L.OP_ATTEND, Q=Q, cap=cache.cap))
    L.csa_attend(dims, cache, qs["q"], W["gamma_q"], W["sink"], q_seq, q_pos, Q,
                 idx if cfg["top_k"] > 0 else None, out, ws)
    torch.cuda.synchronize()
    q = host64(qs["q"])
    qI = qI_host(qs["qI"], cfg) if cfg["top_k"] > 0 else None
    w = host64(qs["w"]) if cfg["top_k"] > 0 else None
    sink = host64(W["sink"]) if W["sink"] is not None else None
    gi = idx.cpu().numpy()
    go = host64(out)
    gs = scores.float().cpu().numpy().astype(np.float64) if scores is not None else None
    per_seq = {}
    stats = []
    lc = logical(cache)
    for i, (b, tau) in enumerate(taus):
        if b not in per_seq:
            per_seq[b] = _oracle_cache(cfg, lc, b)
        entries, ki, raw_of = per_seq[b]
        ne = int(cache.n_entries[b])
        o_ref, sel, sc = R.query_step(tau, q[i], None if qI is None else qI[i], None if w is None else w[i],
                                      None, sink, entries, ki, raw_of, ne, od)
        if cfg["top_k"] > 0:
            V = R.visible_entries(tau, cfg["m"], ne)
            if gs is not None and V and cfg["idx_fmt"] == "mxfp4":
                # BF16 scores: the exact score rounded once to nearest even (within the stated band)
                sc = check_bf16_scores(gs[i, :V], qI[i], w[i], ki[:V], f"bf16 scores seq {b} tau={tau}")
            elif gs is not None and V:
                # scores: float32 accumulation of exact products
                dots = np.abs(ki[:V]) @ np.abs(qI[i]).T
                scale = dots @ np.abs(w[i])
                err = np.abs(gs[i, :V] - sc)
                assert np.all(err <= 1e-5 * scale + 1e-30), f"scores tau={tau}: worst {np.max(err / (scale + 1e-30)):.3g}"
            if not check_topk(gi[i], sc, k, f"{cfg['name']} seq {b} tau={tau}"):
                o_ref = R.query_step(tau, q[i], qI[i], w[i], None, sink, entries, ki, raw_of, ne, od,
                                     sel=gi[i][gi[i] >= 0])[0]
        stats.append(assert_close_q(go[i], o_ref, f"{cfg['name']} out seq {b} tau={tau}"))
    return stats


@pytest.mark.parametrize("idx_fmt", ["e4m3", "mxfp4"])
def test_q_index_topk_attend_small(idx_fmt):
    """Flash dims on a synthetic cache of 5003 entries (ragged tile tail): queries whose
    visible range is empty, below k, not a multiple of 16, and full; windows clipped at 0.
    Indexer keys and queries in E4M3 or MXFP4."""
    cfg = _qcfg(idx_fmt=idx_fmt)
    N = 5003
    tt = [3, 4, 130, 2051, 4 * 700 + 3, 4 * 5003, 4 * 5003 + 77, 4 * 3333 + 1, 9000 * 4]
    taus = list(enumerate(tt))
    dims, cache, qs, W, q_seq, q_pos = _synthetic_decode_setup(
        cfg, len(taus), N, 128, taus, n_entries=[N] * (len(taus) - 1) + [4000])
    _run_index_attend_and_check(cfg, dims, cache, qs, W, q_seq, q_pos, taus)


def test_q_attend_no_sink_and_masked_window():
    """No sink; window ring slots that do not hold the wanted position are skipped."""
    cfg = _qcfg(sink=False)
    taus = [(0, 4 * 600 + 2), (1, 50)]
    dims, cache, qs, W, q_seq, q_pos = _synthetic_decode_setup(cfg, 2, 700, 128, taus, sink=False)
    wp = cache.win_pos.clone()
    wp[0, 5] = -1  # a hole in the ring
    cache.win_pos.copy_(wp)
    _run_index_attend_and_check(cfg, dims, cache, qs, W, q_seq, q_pos, taus)


def test_q_attend_skips_indices_past_visible():
    """A caller's index list holding -1 slots, duplicates and indices at or past the visible
    count V (rows past n_entries hold NaN bytes in every field): only the slots below V count,
    each as one key, and no NaN of a row that is not visible reaches the output."""
    cfg = _qcfg()
    N, k = 3000, cfg["top_k"]
    taus = [(0, 4 * 1500 + 1), (1, 4 * 2999 + 3)]   # V = 1500 (n_entries 2000), V = 2999
    dims, cache, qs, W, q_seq, q_pos = _synthetic_decode_setup(cfg, 2, N, 128, taus, n_entries=[2000, 3000])
    cache.kv.view(2, N, -1)[0, 2000:] = 0xFF          # NaN as E4M3 and as bf16
    rng = np.random.default_rng(5)
    idx = np.empty((2, k), dtype=np.int32)
    for i, (b, tau) in enumerate(taus):
        V = R.visible_entries(tau, cfg["m"], int(cache.n_entries[b]))
        row = rng.choice(V, size=k, replace=False).astype(np.int32)
        bad = rng.choice(k, size=96, replace=False)
        row[bad[:40]] = rng.integers(V, N, size=40)     # invisible (NaN rows for sequence 0)
        row[bad[40:60]] = -1
        row[bad[60:96]] = row[(bad[60:96] + 1) % k]     # duplicates of other slots
        idx[i] = row
    out = torch.zeros((2, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device=DEV)
    ws = _ws(L.csa_workspace_size(dims, L.OP_ATTEND, Q=2, cap=cache.cap))
    L.csa_attend(dims, cache, qs["q"], W["gamma_q"], W["sink"], q_seq, q_pos, 2, _i32(idx), out, ws)
    torch.cuda.synchronize()
    go = host64(out)
    assert np.all(np.isfinite(go))
    od = oracle_dims(cfg)
    q, sink = host64(qs["q"]), host64(W["sink"])
    for i, (b, tau) in enumerate(taus):
        entries, ki, raw_of = _oracle_cache(cfg, cache, b)
        V = R.visible_entries(tau, cfg["m"], int(cache.n_entries[b]))
        sel = idx[i][(idx[i] >= 0) & (idx[i] < V)]
        o_ref = R.query_step(tau, q[i], None, None, None, sink, entries, ki, raw_of, int(cache.n_entries[b]), od,
                             sel=sel)[0]
        assert_close_q(go[i], o_ref, f"past-visible indices seq {b}")


def test_hca_dense_attend_small():
    """HCA dense attention (idx = NULL) over up to 300 entries + the window."""
    cfg = synth.config("c5")
    taus = [(0, 128 * 300 + 5), (1, 127), (2, 128 * 17)]
    dims, cache, qs, W, q_seq, q_pos = _synthetic_decode_setup(cfg, 3, 300, 128, taus)
    _run_index_attend_and_check(cfg, dims, cache, qs, W, q_seq, q_pos, taus)


@pytest.mark.parametrize("idx_fmt,paged", [("e4m3", False), ("mxfp4", False), ("e4m3", True), ("mxfp4", True)])
def test_q_forward_end_to_end(idx_fmt, paged):
    """Compress a 600-token prefix in chunks, then a 96-token forward chunk (compress +
    index + top-k + attend) on 2 sequences; the oracle builds its own cache from the same
    hidden states.  Queries whose selection differs only through ties or a stored-code flip
    are checked for validity on the GPU's selection.  The chunk's queries take the tiled
    (prefill) indexer, with E4M3 or MXFP4 keys; the cache is contiguous or paged (128-token
    pages in a shuffled pool)."""
    cfg = _qcfg(idx_fmt=idx_fmt)
    dims = L.Dims.from_config(cfg)
    od = oracle_dims(cfg)
    B, n0, T = 2, 600, 96
    k = cfg["top_k"]
    W = synth.weights(cfg, seed=21, device=DEV)
    Hs = torch.stack([synth.hidden(cfg, b, 0, n0 + T, seed=21, device=DEV) for b in range(B)])
    cache = paged_cache(dims, B, 256, T + 128, seed=21) if paged else L.Cache(dims, B=B, cap=256, win_cap=T + 128)
    _compress_chunks(dims, W, cache, Hs[:, :n0].contiguous(), [256, 3, 341])
    qs = synth.queries(cfg, B * T, seed=21, device=DEV)
    out = torch.zeros((B * T, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((B * T, k), dtype=torch.int32, device=DEV)
    ws = _ws(L.csa_workspace_size(dims, L.OP_FORWARD, B=B, T=T, cap=cache.cap))
    L.csa_forward(dims, lib_weights(W, True), cache, Hs[:, n0:].contiguous(), T, _i32([n0] * B),
                  qs["q"], qs["qI"], qs["w"], W["gamma_q"], W["sink"], out, idx, ws)
    torch.cuda.synchronize()
    cache = logical(cache)
    OW = oracle_weights(W)
    q, qI, w = host64(qs["q"]), qI_host(qs["qI"], cfg), host64(qs["w"])
    sink = host64(W["sink"])
    gi, go = idx.cpu().numpy(), host64(out)
    for b in range(B):
        comp = R.compress_sequence(host64(Hs[b]), OW, od)
        _check_cache_vs_oracle(cfg, cache, b, comp, n0 + T, f"e2e seq {b}")
        g_entries = decode_rows(cache.kv[b].cpu().numpy(), cfg)
        g_ki = keys_of(cache, b, 0, cache.cap, cfg)
        nb = (n0 + T) // cfg["m"]
        for t in range(T):
            i = b * T + t
            tau = n0 + t
            o_ref, sel, sc = R.query_step(tau, q[i], qI[i], w[i], None, sink, comp["entry"], comp["ki"],
                                          lambda p: comp["raw"][p], nb, od)
            try:
                same = check_topk(gi[i], sc, k, f"e2e seq {b} tau={tau}")
            except AssertionError:
                # allowed only if the GPU's selection is the exact top-k of the scores its own
                # (validated, flip-only) stored keys give
                V = R.visible_entries(tau, cfg["m"], nb)
                sc_g = R.scores_for_topk(qI[i], w[i], g_ki[:V], od)
                same = check_topk(gi[i], sc_g, k, f"e2e seq {b} tau={tau} (GPU keys)")
                same = False
            if not same:
                sel_g = gi[i][gi[i] >= 0]
                keys = np.concatenate([g_entries[sel_g], comp["raw"][R.window_positions(tau, cfg["n_win"])]])
                o_ref = R.attend(q[i], tau, keys, None, sink, od)
            assert_close_q(go[i], o_ref, f"e2e out seq {b} tau={tau}")


@pytest.mark.parametrize("idx_fmt,paged", [("e4m3", False), ("mxfp4", False), ("mxfp4", True)])
def test_q_forward_decode_steps(idx_fmt, paged):
    """Nine one-token forward steps (tau = 600 .. 608, two of them completing an entry) on a
    cache whose capacity spans two top-k segments: the path that scores before compressing
    and runs the projection step inside the top-k threshold launch.  Outputs, selections and
    the cache afterwards are checked against the oracle as in the chunked test; the cache is
    contiguous or paged."""
    cfg = _qcfg(idx_fmt=idx_fmt)
    dims = L.Dims.from_config(cfg)
    od = oracle_dims(cfg)
    B, n0, steps = 2, 600, 9
    k = cfg["top_k"]
    W = synth.weights(cfg, seed=23, device=DEV)
    lw = lib_weights(W, True)
    Hs = torch.stack([synth.hidden(cfg, b, 0, n0 + steps, seed=23, device=DEV) for b in range(B)])
    cache = paged_cache(dims, B, 16384, 128, seed=23) if paged else L.Cache(dims, B=B, cap=16384, win_cap=128)
    _compress_chunks(dims, W, cache, Hs[:, :n0].contiguous(), [256, 344])
    qs = synth.queries(cfg, B * steps, seed=23, device=DEV)
    ws = _ws(L.csa_workspace_size(dims, L.OP_FORWARD, B=B, T=1, cap=cache.cap))
    outs, idxs = [], []
    for t in range(steps):
        rows = [b * steps + t for b in range(B)]
        out = torch.zeros((B, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device=DEV)
        idx = torch.zeros((B, k), dtype=torch.int32, device=DEV)
        L.csa_forward(dims, lw, cache, Hs[:, n0 + t:n0 + t + 1].contiguous(), 1, _i32([n0 + t] * B),
                      qs["q"][rows].contiguous(), qs["qI"][rows].contiguous(), qs["w"][rows].contiguous(),
                      W["gamma_q"], W["sink"], out, idx, ws)
        outs.append(out)
        idxs.append(idx)
    torch.cuda.synchronize()
    cache = logical(cache)
    OW = oracle_weights(W)
    q, qI, w = host64(qs["q"]), qI_host(qs["qI"], cfg), host64(qs["w"])
    sink = host64(W["sink"])
    for b in range(B):
        comp = R.compress_sequence(host64(Hs[b]), OW, od)
        _check_cache_vs_oracle(cfg, cache, b, comp, n0 + steps, f"decode steps seq {b}")
        g_entries = decode_rows(cache.kv[b].cpu().numpy(), cfg)
        g_ki = keys_of(cache, b, 0, cache.cap, cfg)
        nb = (n0 + steps) // cfg["m"]
        for t in range(steps):
            i = b * steps + t
            tau = n0 + t
            gi = idxs[t][b].cpu().numpy()
            go = host64(outs[t][b:b + 1])[0]
            o_ref, sel, sc = R.query_step(tau, q[i], qI[i], w[i], None, sink, comp["entry"], comp["ki"],
                                          lambda p: comp["raw"][p], nb, od)
            try:
                same = check_topk(gi, sc, k, f"decode seq {b} tau={tau}")
            except AssertionError:
                V = R.visible_entries(tau, cfg["m"], nb)
                sc_g = R.scores_for_topk(qI[i], w[i], g_ki[:V], od)
                same = check_topk(gi, sc_g, k, f"decode seq {b} tau={tau} (GPU keys)")
                same = False
            if not same:
                sel_g = gi[gi >= 0]
                keys = np.concatenate([g_entries[sel_g], comp["raw"][R.window_positions(tau, cfg["n_win"])]])
                o_ref = R.attend(q[i], tau, keys, None, sink, od)
            assert_close_q(go, o_ref, f"decode out seq {b} tau={tau}")


@pytest.mark.parametrize("paged", [False, True])
def test_hca_forward_decode_steps(paged):
    """Eight one-token forward steps of an HCA layer (m' = 128, tau = 250 .. 257 on 2
    sequences; the step at 255 completes entry 1 and the next ones attend over it): the path
    whose fold runs inside the attention launch, the attention workgroups finalizing the new
    token's window row themselves.  Outputs and the cache afterwards against the oracle."""
    cfg = synth.config("c5")
    dims = L.Dims.from_config(cfg)
    od = oracle_dims(cfg)
    B, n0, steps = 2, 250, 8
    W = synth.weights(cfg, seed=29, device=DEV)
    lw = lib_weights(W, False)
    Hs = torch.stack([synth.hidden(cfg, b, 0, n0 + steps, seed=29, device=DEV) for b in range(B)])
    cache = paged_cache(dims, B, 8, 128, seed=29) if paged else L.Cache(dims, B=B, cap=8, win_cap=128)
    _compress_chunks(dims, W, cache, Hs[:, :n0].contiguous(), [100, 150])
    qs = synth.queries(cfg, B * steps, seed=29, device=DEV)
    ws = _ws(L.csa_workspace_size(dims, L.OP_FORWARD, B=B, T=1, cap=cache.cap))
    outs = []
    for t in range(steps):
        print(f"hca forward step tau={n0 + t} paged={paged}", flush=True)
        rows = [b * steps + t for b in range(B)]
        out = torch.zeros((B, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device=DEV)
        L.csa_forward(dims, lw, cache, Hs[:, n0 + t:n0 + t + 1].contiguous(), 1, _i32([n0 + t] * B),
                      qs["q"][rows].contiguous(), None, None, W["gamma_q"], W["sink"], out, None, ws)
        outs.append(out)
    torch.cuda.synchronize()
    cache = logical(cache)
    OW = oracle_weights(W)
    q, sink = host64(qs["q"]), host64(W["sink"])
    nb = (n0 + steps) // cfg["m"]
    for b in range(B):
        comp = R.compress_sequence(host64(Hs[b]), OW, od)
        _check_cache_vs_oracle(cfg, cache, b, comp, n0 + steps, f"hca decode steps seq {b}")
        for t in range(steps):
            tau = n0 + t
            o_ref = R.query_step(tau, q[b * steps + t], None, None, None, sink, comp["entry"], None,
                                 lambda p: comp["raw"][p], nb, od)[0]
            assert_close_q(host64(outs[t][b:b + 1])[0], o_ref, f"hca decode out seq {b} tau={tau}")


@pytest.mark.parametrize("idx_fmt", ["e4m3", "mxfp4"])
def test_index_scores_grouped_equals_plain(idx_fmt):
    """csa_index_scores_grouped (key tiles shared by 16 queries of one sequence, the prefill
    kernel) gives the scores of csa_index_scores bit for bit: 48 queries in three groups over
    two sequences of 3001 entries (ragged tail), positions spread so the visible counts differ
    within a group."""
    cfg = _qcfg(idx_fmt=idx_fmt)
    N = 3001
    seqs = [0] * 32 + [1] * 16
    taus = [(b, 4 * 100 + 97 * i) for i, b in enumerate(seqs)]
    dims, cache, qs, W, q_seq, q_pos = _synthetic_decode_setup(cfg, 2, N, 128, taus, seed=13)
    Q = len(taus)
    sdt = torch.bfloat16 if idx_fmt == "mxfp4" else torch.float32
    a = torch.zeros((Q, N), dtype=sdt, device=DEV)
    b = torch.zeros((Q, N), dtype=sdt, device=DEV)
    L.csa_index_scores(dims, cache, qs["qI"], qs["w"], q_seq, q_pos, Q, a, N)
    L.csa_index_scores_grouped(dims, cache, qs["qI"], qs["w"], q_seq, q_pos, Q, b, N)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16) if idx_fmt == "mxfp4" else a.view(torch.int32),
                       b.view(torch.int16) if idx_fmt == "mxfp4" else b.view(torch.int32))


def test_deterministic_repeat():
    """Two runs of index + top-k + attend on the same inputs give identical bits."""
    cfg = _qcfg()
    taus = [(0, 4 * 3000), (1, 4 * 2999 + 3)]
    dims, cache, qs, W, q_seq, q_pos = _synthetic_decode_setup(cfg, 2, 3000, 128, taus)
    outs = []
    for _ in range(2):
        idx = torch.zeros((2, cfg["top_k"]), dtype=torch.int32, device=DEV)
        out = torch.zeros((2, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device=DEV)
        L.csa_index_topk(dims, cache, qs["qI"], qs["w"], q_seq, q_pos, 2, idx, None,
                         _ws(L.csa_workspace_size(dims, L.OP_INDEX_TOPK, Q=2, cap=3000)))
        L.csa_attend(dims, cache, qs["q"], W["gamma_q"], W["sink"], q_seq, q_pos, 2, idx, out,
                     _ws(L.csa_workspace_size(dims, L.OP_ATTEND, Q=2, cap=3000)))
        torch.cuda.synchronize()
        outs.append((idx.cpu().clone(), out.view(torch.int16).cpu().clone()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


# ----------------------------------------------------------------------------- full sizes


def _decode_full(name, B=None, check_scores_for=2, paged=False, **over):
    """A decode step of a full-size configuration on a synthetic cache: every query's
    selection (under the tie rule) and output are checked against the oracle."""
    cfg = synth.config(name, **over)
    B = B or cfg["B"]
    N = cfg["prefix"] // cfg["m"]
    tau = cfg["prefix"]
    taus = [(b, tau) for b in range(B)]
    dims, cache, qs, W, q_seq, q_pos = _synthetic_decode_setup(cfg, B, N, cfg["n_win"], taus, seed=31, paged=paged)
    stats = _run_index_attend_and_check(cfg, dims, cache, qs, W, q_seq, q_pos, taus,
                                        check_scores=True)
    return stats


def test_c2_decode_full_size():
    """Flash decode, 16 sequences x 32768 entries, k=512: the bench's kernels and grid."""
    _decode_full("c2")


def test_c2_decode_full_size_mxfp4():
    """The same with the indexer's keys and queries in MXFP4."""
    _decode_full("c2", idx_fmt="mxfp4")


def test_c3_decode_full_size():
    """Pro decode, 4 sequences x 262144 entries (1M tokens), 128 heads, k=1024 (segmented
    top-k with a merge stage)."""
    _decode_full("c3")


def test_c3_decode_full_size_mxfp4():
    """The same with MXFP4 indexer keys and queries: bfloat16 score rows of 262144 entries
    through the threshold and final passes with k = 1024."""
    _decode_full("c3", idx_fmt="mxfp4")


def test_c5_hca_decode_full_size():
    """HCA decode, 8 sequences x 8192 entries (1M tokens, m'=128), dense attention."""
    _decode_full("c5")


def test_c2_decode_full_size_paged():
    """Flash decode at full size on a paged cache: 128-token pages (32 entries) in a shuffled
    pool, one block table per sequence."""
    _decode_full("c2", paged=True)


def test_c2_decode_full_size_mxfp4_paged():
    """The same with MXFP4 keys (per page: 32 rows of element bytes, then 32 rows of scales)."""
    _decode_full("c2", idx_fmt="mxfp4", paged=True)


def test_c3_decode_full_size_paged():
    """Pro decode at full size on a paged cache (8192 pages per sequence)."""
    _decode_full("c3", paged=True)


def test_c5_hca_decode_full_size_paged():
    """HCA dense decode on a paged cache: a 128-token page holds one HCA entry, so every
    entry is looked up in the block table."""
    _decode_full("c5", paged=True)


def _prefill_sample(T, m, seed=0):
    """256 query rows of a T-token chunk: the first and last 32, 32 at positions = 0 and 32 at
    positions = m - 1 (mod m) spread over the chunk, and 128 more drawn at random."""
    rng = np.random.default_rng(seed)
    first, last = list(range(32)), list(range(T - 32, T))
    mid = np.arange(32, T - 32)
    at0 = rng.choice(mid[mid % m == 0], 32, replace=False).tolist()
    at3 = rng.choice(mid[mid % m == m - 1], 32, replace=False).tolist()
    rest = np.setdiff1d(mid, at0 + at3)
    return sorted(set(first + last + at0 + at3 + rng.choice(rest, 128, replace=False).tolist()))


@pytest.mark.parametrize("name,idx_fmt", [("c4a", "e4m3"), ("c4a", "mxfp4"), ("c4b", "e4m3"), ("mid", "e4m3"),
                                           ("mid_ties", "e4m3")])
def test_c4_prefill_full_size_sampled(name, idx_fmt):
    """Flash chunked prefill at full size: a 32768-token chunk after a 1048576-token prefix
    (c4a: 262144 entries) or a 262144-token prefix (c4b: 65536 entries).  The prefix cache,
    its window ring and the projection state of the block before the chunk (zeros) are inputs
    given to both sides; csa_forward compresses the chunk (8192 new entries), scores every
    query against all visible entries, selects 512 and attends.  256 stratified query rows of
    the chunk are checked against the oracle, which folds the chunk's entries from the same
    hidden states; every new entry and key is checked.  Indexer keys in E4M3 or MXFP4.
    mid: a 256-token chunk after a 48000-token prefix (about 12000 visible entries, every row
    checked), where the prefill indexer's own threshold splits each row over 16 segments;
    mid_ties: the same with every prefix key equal, so that every query's prefix scores tie
    at the threshold and the candidates overflow into the whole-row selection."""
    base = {"mid": "c4b", "mid_ties": "c4b"}.get(name, name)
    cfg = dict(synth.config(base), idx_fmt=idx_fmt)
    if base != name:
        cfg.update(prefix=48000, T=256)
    dims = L.Dims.from_config(cfg)
    od = oracle_dims(cfg)
    m, k, T, p0 = cfg["m"], cfg["top_k"], cfg["T"], cfg["prefix"]
    N0 = p0 // m
    cap = (p0 + T) // m
    R_win = T + cfg["n_win"]
    taus0 = [(0, p0 - 1)]
    dims, cache, _, _, _, _ = _synthetic_decode_setup(cfg, 1, cap, R_win, taus0, seed=41,
                                                      n_entries=[N0])
    cache.state.zero_()
    if name == "mid_ties":
        cache.ki[0, :N0] = cache.ki[0, :1].clone()
    W = synth.weights(cfg, seed=41, device=DEV)
    H = synth.hidden(cfg, 0, p0, p0 + T, seed=41, device=DEV)
    qs = synth.queries(cfg, T, seed=41, device=DEV, tag="prefill")
    out = torch.zeros((T, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    # inputs both sides see: prefix entries, keys and ring rows (before the chunk overwrites)
    prefix_entries = decode_rows(cache.kv[0, :N0].cpu().numpy(), cfg)
    prefix_ki = keys_of(cache, 0, 0, N0, cfg)
    ring = decode_rows(cache.win[0].cpu().numpy(), cfg)
    ring_pos = cache.win_pos[0].cpu().numpy()
    ws = _ws(L.csa_workspace_size(dims, L.OP_FORWARD, B=1, T=T, cap=cap, q_chunk=4096))
    L.csa_forward(dims, lib_weights(W, True), cache, H.unsqueeze(0).contiguous(), T,
                  _i32([p0]), qs["q"], qs["qI"], qs["w"], W["gamma_q"], W["sink"], out, idx, ws)
    torch.cuda.synchronize()
    assert int(cache.n_entries[0]) == cap

    # oracle: the chunk's projections, entries (first block's b rows = the given zero state)
    OW = oracle_weights(W)
    Hn = host64(H)
    P = {p: R.project(Hn, OW[p]) for p in ("kv_a", "kv_b", "z_a", "z_b", "ki_a", "ki_b", "zi_a", "zi_b")}
    zc = np.zeros((m, cfg["c"]))
    zi = np.zeros((m, cfg["c_I"]))
    pre = R.csa_fold(P["kv_a"], P["kv_b"], P["z_a"], P["z_b"], OW["B_a"], OW["B_b"], m, prev_b=(zc, zc))
    kpre = R.csa_fold(P["ki_a"], P["ki_b"], P["zi_a"], P["zi_b"], OW["BI_a"], OW["BI_b"], m, prev_b=(zi, zi))
    fin = R.finalize_kv(pre, m * (N0 + np.arange(T // m)), OW["gamma_kv"], od)
    ent_new, _ = R.store_kv(fin, od)
    ki_new, _ = R.store_index_keys(kpre, od)
    raw_fin = R.finalize_kv(P["kv_a"], p0 + np.arange(T), OW["gamma_kv"], od)
    raw_new, _ = R.store_kv(raw_fin, od)
    # the GPU's new entries/keys/rows against the oracle's (storage rounding rule)
    g_new = decode_rows(cache.kv[0, N0:cap].cpu().numpy(), cfg)
    c, r = cfg["c"], cfg["rope_dim"]
    check_stored_codes(g_new[:, :c - r], fin[:, :c - r], "e4m3", "c4 new entries/nope")
    check_stored_codes(g_new[:, c - r:], fin[:, c - r:], "bf16", "c4 new entries/rope")
    g_ki_new = keys_of(cache, 0, N0, cap, cfg)
    if idx_fmt == "mxfp4":
        check_stored_mxfp4(cache.ki_codes[0, N0:cap].cpu().numpy(), cache.ki_scales[0, N0:cap].cpu().numpy(),
                           kpre, "c4 new keys")
    else:
        check_stored_codes(g_ki_new, kpre, "e4m3", "c4 new keys")
    entries = np.concatenate([prefix_entries, ent_new])
    ki = np.concatenate([prefix_ki, ki_new])
    g_entries = np.concatenate([prefix_entries, g_new])
    g_ki = np.concatenate([prefix_ki, g_ki_new])

    def raw_of(pos):
        pos = np.asarray(pos)
        old = pos < p0
        rows = np.empty((len(pos), cfg["c"]))
        slots = pos[old] % R_win
        assert np.all(ring_pos[slots] == pos[old])
        rows[old] = ring[slots]
        rows[~old] = raw_new[pos[~old] - p0]
        return rows

    q, qI, w = host64(qs["q"]), qI_host(qs["qI"], cfg), host64(qs["w"])
    sink = host64(W["sink"])
    gi, go = idx.cpu().numpy(), host64(out)
    for t in _prefill_sample(T, m):
        tau = p0 + t
        o_ref, sel, sc = R.query_step(tau, q[t], qI[t], w[t], None, sink, entries, ki, raw_of, cap, od)
        try:
            same = check_topk(gi[t], sc, k, f"c4 t={t}")
        except AssertionError:
            V = R.visible_entries(tau, m, cap)
            check_topk(gi[t], R.scores_for_topk(qI[t], w[t], g_ki[:V], od), k,
                       f"c4 t={t} (GPU keys)")
            same = False
        if not same:
            sel_g = gi[t][gi[t] >= 0]
            keys = np.concatenate([g_entries[sel_g], raw_of(R.window_positions(tau, cfg["n_win"]))])
            o_ref = R.attend(q[t], tau, keys, None, sink, od)
        assert_close_q(go[t], o_ref, f"c4 out t={t}")


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_topk_exact_on_crafted_scores(fmt):
    """csa_topk on given scores must equal the oracle's selection exactly (same input bits):
    heavy ties (integer scores), -0/+0, scores rising or falling with the index (every
    candidate in one segment), rows shorter than k, exactly k, k + 1, ragged segment tails,
    rows one workgroup selects from (33000 and 65536 entries) and longer ones (90001 entries,
    k = 1024).  Ties and -0/+0 rows defeat the sampled
    threshold, so they also exercise the exact whole-row fallback.  float32 rows, and the
    bfloat16 rows of the MXFP4 indexer path (whose rounding turns the slow ramps into runs of
    equal scores)."""
    for k, cap in ((1024, 90001), (512, 4096), (8, 37), (512, 33000), (2048, 65536)):
        cfg = _qcfg(top_k=k, idx_fmt="mxfp4" if fmt == "bf16" else "e4m3")
        dims = L.Dims.from_config(cfg)
        m = cfg["m"]
        Vs = sorted({0, 1, min(k, cap), min(k + 1, cap), cap // 3, cap - 5, cap})
        Q = len(Vs) * 5
        cache = L.Cache(dims, B=1, cap=cap, win_cap=128)
        cache.n_entries.fill_(cap)
        rng = np.random.default_rng(k + cap)
        sc = np.zeros((Q, cap), dtype=np.float32)
        pos = []
        for i in range(Q):
            V = Vs[i // 5]
            kind = i % 5
            if kind == 0:
                sc[i] = rng.standard_normal(cap).astype(np.float32)
            elif kind == 1:
                sc[i] = rng.integers(-3, 4, cap).astype(np.float32)
            elif kind == 2:
                sc[i] = np.where(rng.random(cap) < 0.5, -0.0, 0.0).astype(np.float32)
                sc[i, rng.integers(0, cap, 5)] = 1.0
            elif kind == 3:
                sc[i] = (np.arange(cap) * 1e-3 + rng.random(cap) * 1e-4).astype(np.float32)
            else:
                sc[i] = (-np.arange(cap) * 1e-3).astype(np.float32)
            pos.append(m * V + (i % m))
        scores = torch.from_numpy(sc).to(DEV)
        if fmt == "bf16":
            scores = scores.to(torch.bfloat16)
            sc = scores.float().cpu().numpy()
        idx = torch.full((Q, k), -7, dtype=torch.int32, device=DEV)
        ws = _ws(L.csa_topk_workspace_size(dims, Q, cap))
        L.csa_topk(dims, cache, _i32([0] * Q), _i32(pos), Q, scores, cap, idx, ws)
        torch.cuda.synchronize()
        gi = idx.cpu().numpy()
        for i in range(Q):
            V = Vs[i // 5]
            ref = R.topk(sc[i, :V].astype(np.float64), k)
            got = gi[i][gi[i] >= 0]
            assert np.array_equal(got, ref), f"k={k} cap={cap} V={V} kind={i % 5}"
            assert np.all(gi[i][len(got):] == -1)


@pytest.mark.parametrize("N,taus", [(20000, "mixed"), (5003, "short"), (70000, "long")])
def test_index_topk_grouped_equals_ungrouped(N, taus):
    """csa_index_topk_grouped (the prefill indexer that thresholds its own scores, then the
    selection from its lists) selects exactly what csa_index_topk does, with the same scores:
    two sequences of 48 queries each (3 groups of 16), positions consecutive within a
    sequence; visible counts below and above the threshold's 8192 (every score a candidate,
    or a sampled threshold), rows split over several segments."""
    cfg = _qcfg()
    dims = L.Dims.from_config(cfg)
    m, k = cfg["m"], cfg["top_k"]
    start = {"mixed": [4 * 6000, 4 * 19000], "short": [4 * 3000, 4 * 4900], "long": [4 * 60000, 4 * 69000]}[taus]
    Qs = 48
    pos = [s0 + t for s0 in start for t in range(Qs)]
    seqs = [b for b in range(2) for _ in range(Qs)]
    dims, cache, qs, W, q_seq, q_pos = _synthetic_decode_setup(cfg, 2, N, 128, list(zip(seqs, pos)), seed=17)
    Q = len(pos)
    out = []
    for fn in (L.csa_index_topk, L.csa_index_topk_grouped):
        idx = torch.full((Q, k), -7, dtype=torch.int32, device=DEV)
        sc = torch.zeros((Q, N), dtype=torch.float32, device=DEV)
        ws = _ws(L.csa_workspace_size(dims, L.OP_INDEX_TOPK, Q=Q, cap=N))
        fn(dims, cache, qs["qI"], qs["w"], q_seq, q_pos, Q, idx, sc, ws)
        torch.cuda.synchronize()
        out.append((idx.cpu(), sc.cpu()))
    for i in range(Q):
        V = R.visible_entries(pos[i], m, N)
        assert torch.equal(out[0][1][i, :V], out[1][1][i, :V]), f"scores row {i}"
        assert torch.equal(out[0][0][i], out[1][0][i]), f"selection row {i} (V={V})"


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_topk_exact_many_long_rows(fmt):
    """Enough long rows that each threshold workgroup filters several segments against one
    sample (400 rows x 11 segments of 8192, the last group of segments ragged): random rows,
    integer ties and falling ramps (the whole-row fallback), visible counts from k to the row
    length.  The selection must equal the oracle's exactly."""
    k, cap, Q = 512, 90001, 400
    cfg = _qcfg(top_k=k, idx_fmt="mxfp4" if fmt == "bf16" else "e4m3")
    dims = L.Dims.from_config(cfg)
    m = cfg["m"]
    cache = L.Cache(dims, B=1, cap=cap, win_cap=128)
    cache.n_entries.fill_(cap)
    rng = np.random.default_rng(77)
    sc = rng.standard_normal((Q, cap)).astype(np.float32)
    sc[1::7] = rng.integers(-3, 4, (len(range(1, Q, 7)), cap)).astype(np.float32)
    sc[3::11] = -np.arange(cap, dtype=np.float32) * 1e-3
    Vs = rng.integers(k, cap + 1, Q)
    Vs[:4] = [k, k + 1, cap - 1, cap]
    pos = [int(m * V + (i % m)) for i, V in enumerate(Vs)]
    scores = torch.from_numpy(sc).to(DEV)
    if fmt == "bf16":
        scores = scores.to(torch.bfloat16)
        sc = scores.float().cpu().numpy()
    idx = torch.full((Q, k), -7, dtype=torch.int32, device=DEV)
    ws = _ws(L.csa_topk_workspace_size(dims, Q, cap))
    L.csa_topk(dims, cache, _i32([0] * Q), _i32(pos), Q, scores, cap, idx, ws)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    for i in range(Q):
        ref = R.topk(sc[i, :Vs[i]].astype(np.float64), k)
        assert np.array_equal(gi[i], ref), f"row {i} V={Vs[i]}"
