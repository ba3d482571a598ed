"""Benchmark of the compressed sparse attention path on one MI355X.

Default workload (the reported line): Flash-shaped CSA decode, config c2 -- 16 sequences,
each with a 131072-token context already compressed into 32768 entries (m = 4); d = 4096,
64 query heads of 512 (RoPE on the last 64), indexer 64 heads x 128, top-k 512, window 128,
sink per head; KV rows E4M3 + bf16 RoPE dims, indexer keys E4M3.  The cache is built untimed
by compressing synthetic hidden states N(0,1) with weights N(0, 1/4096).

One decode step = the whole path for one new token per sequence: compress the token
(projection GEMM, window row, projection state; an entry when a block completes), indexer
scores over the visible entries, top-k, attention over the selected entries + window rows.
Several copies of the cache rotate between steps so every step reads its cache from HBM rather
than from the 256 MB Infinity Cache.  The steps run from captured HIP graphs, each holding one
cycle of steps over the copies back to back (a decode loop captured once, as a serving loop over
layers would be), so a graph launch is paid once per cycle rather than once per step.

Other workloads (--config): c3 (Pro decode, 4 x 1M tokens), c5 (HCA decode, 8 x 1M tokens),
c4a / c4b (32768-token prefill chunk after a 1M- / 262144-token prefix; one step = one
csa_forward of the chunk), c1 (tiny fp32 prefill); c2fp4, c4afp4 and c4bfp4 are c2, c4a and
c4b with the indexer's keys and queries in MXFP4.

Per-kernel durations: each kernel of the step is also launched 20 times back to back inside
one graph (same inputs, same grid), timed with HIP events around the replay; the dominant
kernel's average gives the roofline line.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12        # bytes/s, MI355X HBM3E
BF16_PEAK = 2.5e15       # dense bf16 MFMA FLOP/s
FP8_PEAK = 5.0e15        # dense fp8 MFMA FLOP/s
FP4_PEAK = 10.1e15       # dense fp4 (MXFP4) MFMA FLOP/s
MALL_BYTES = 256 << 20   # MI355X last-level (Infinity) cache
CAL_BYTES = 256 << 20    # plain device copy that calibrates the FETCH_SIZE / WRITE_SIZE counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_c2_traffic.txt")
INDEXER_SRC = os.path.join(ROOT, "long_context_attention_11_amd", "csrc", "indexer.hip")


def code_digest(path):
    """sha256 of a C++/HIP source with its comments and blank lines removed and each line
    stripped: a change to the code changes it, a change to a comment does not."""
    import hashlib
    import re
    src = open(path, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    code = "\n".join(l.strip() for l in src.splitlines() if l.strip())
    return hashlib.sha256(code.encode()).hexdigest()


def measured_traffic():
    """HBM bytes per indexer launch from the committed counter summary, or None when the
    indexer's code changed since the counters were taken (the summary records its digest)."""
    try:
        kv = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line)
    except OSError:
        return None
    if kv.get("indexer_code_sha256", "").strip() != code_digest(INDEXER_SRC):
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def calibration_copy():
    """One plain device-to-device copy of CAL_BYTES (its counters scale the indexer's)."""
    import torch
    src = torch.ones(CAL_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--layer", action="store_true",
                    help="time the whole attention layer: the query-side projections before the path "
                         "and the grouped output projection after it included (bf16 configurations)")
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c2fp4", "c3", "c4a", "c4afp4", "c4b", "c4bfp4", "c5",
                                                       "c6", "c6fp4"])
    ap.add_argument("--copies", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--paged", action="store_true",
                    help="decode on a paged cache (128-token pages dealt over a shuffled pool)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-extra", action="store_true",
                    help="with the default c2 workload, skip the c3 decode, c4a prefill and batch-series runs")
    return ap.parse_args()


def lib_weights(L, W, dual):
    import torch
    if W.get("w_ik") is not None:   # CSA2: single path, no bias, entry-to-key projection
        return L.Weights(torch.stack([W["kv"], W["z"]]).contiguous(), None, W["w_ik"].contiguous(), None,
                         W["gamma_kv"])
    if dual:
        return L.Weights(torch.stack([W["kv_a"], W["kv_b"], W["z_a"], W["z_b"]]).contiguous(),
                         torch.stack([W["B_a"], W["B_b"]]).contiguous(),
                         torch.stack([W["ki_a"], W["ki_b"], W["zi_a"], W["zi_b"]]).contiguous(),
                         torch.stack([W["BI_a"], W["BI_b"]]).contiguous(), W["gamma_kv"])
    return L.Weights(torch.stack([W["kv"], W["z"]]).contiguous(), W["B"].contiguous(), None, None,
                     W["gamma_kv"])


PAGE_TOKENS = 128   # one page holds 32 CSA entries or 1 HCA entry


def build_cache(L, synth, cfg, dims, lw, dev, B, n_tokens, cap, win_cap, chunk=8192, paged=False):
    """Compress n_tokens synthetic tokens of each sequence into a fresh cache (untimed).
    Paged: every sequence's pages are dealt at random over one pool (a seeded permutation)."""
    import torch
    if paged:
        E = PAGE_TOKENS // cfg["m"]
        mb = -(-cap // E)
        perm = torch.randperm(B * mb, generator=torch.Generator().manual_seed(7)).to(torch.int32)
        cache = L.Cache(dims, B=B, cap=cap, win_cap=win_cap, device=dev, block_table=perm.view(B, mb).to(dev),
                        page_tokens=PAGE_TOKENS, n_pages=B * mb)
    else:
        cache = L.Cache(dims, B=B, cap=cap, win_cap=win_cap, device=dev)
    chunk = min(chunk, n_tokens)
    ws = torch.empty(max(1, L.csa_workspace_size(dims, L.OP_COMPRESS, B=B, T=chunk)), dtype=torch.uint8, device=dev)
    for t0 in range(0, n_tokens, chunk):
        T = min(chunk, n_tokens - t0)
        H = torch.stack([synth.hidden(cfg, b, t0, t0 + T, device=dev) for b in range(B)])
        L.csa_compress(dims, lw, cache, H, T, torch.full((B,), t0, dtype=torch.int32, device=dev), ws)
        del H
    torch.cuda.synchronize()
    return cache


def clone_cache(c):
    import copy
    d = copy.copy(c)
    for k in ("kv", "ki", "n_entries", "win", "win_pos", "state"):
        v = getattr(c, k)
        setattr(d, k, None if v is None else v.clone())
    return d


def capture(fn):
    """Capture fn() (HIP launches on the current stream) into a graph; return its replay."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def kernel_time_us(fns, reps=20, rounds=5):
    """Average duration of one launch: `reps` launches (cycling through fns) captured back to
    back in one graph, HIP events around each replay; the median round is kept."""
    import torch
    g = capture(lambda: [fns[i % len(fns)]() for i in range(reps)])
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / reps)
    times.sort()
    return times[len(times) // 2]


# ----------------------------------------------------------------------------- CPU baseline


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where it is not readable)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_keys_and_queries(cfg, sc, qs, N):
    """Indexer keys of sequence 0 and the indexer queries, decoded as the oracle reads them
    (E4M3, or MXFP4 element codes and block scales)."""
    import numpy as np

    from oracle import codecs
    if cfg["idx_fmt"] == "mxfp4":
        cI, nh = cfg["c_I"], cfg["n_hI"]
        kb = sc["ki"][0].numpy()
        ki = codecs.mxfp4_decode(kb[:N * cI // 2].reshape(N, cI // 2), kb[N * cI // 2:].reshape(N, cI // 32))
        qb = qs["qI"].numpy()
        Q = qb.shape[0]
        qI = codecs.mxfp4_decode(qb[:, :nh * cI // 2].reshape(Q, nh, cI // 2),
                                 qb[:, nh * cI // 2:].reshape(Q, nh, cI // 32))
        return ki, qI
    if cfg["idx_fmt"] == "f32":
        return sc["ki"][0].numpy().astype(np.float64), qs["qI"].float().numpy().astype(np.float64)
    return codecs.e4m3_decode(sc["ki"][0].numpy()), codecs.e4m3_decode(qs["qI"].numpy())


def cpu_baseline(cfg, seconds):
    """The oracle, untuned, on a bounded sample of the same decode step: single queries
    (compress of the new token: every projection and its window row; indexer over all visible
    entries; top-k; attention), synthetic inputs of the workload's shapes."""
    import numpy as np

    import synth
    from oracle import codecs
    from oracle import csa_ref as R

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    idx = cfg["top_k"] > 0
    od = R.Dims(d=cfg["d"], c=cfg["c"], rope_dim=cfg["rope_dim"], n_h=cfg["n_h"], c_I=cfg["c_I"],
                n_hI=cfg["n_hI"], m=cfg["m"], dual=cfg["dual"], top_k=cfg["top_k"],
                n_win=cfg["n_win"], kv_fmt=cfg["kv_fmt"], idx_fmt=cfg["idx_fmt"] if idx else "e4m3")
    N = cfg["prefix"] // cfg["m"]
    tau = cfg["prefix"]
    W = synth.weights(cfg, device="cpu")
    OW = {k: (None if v is None else v.float().numpy().astype(np.float64)) for k, v in W.items()
          if k not in ("gamma_q", "sink")}
    sink = W["sink"].numpy().astype(np.float64)
    sc = synth.synthetic_cache(cfg, 1, N, cfg["n_win"], device="cpu")
    c, r = cfg["c"], cfg["rope_dim"]

    def dec(b):
        if cfg["kv_fmt"] == "q4":   # bf16 RoPE dims, MXFP4 element bytes and scale codes
            ne = (c - r) // 2
            return np.concatenate([codecs.mxfp4_decode(b[:, 2 * r:2 * r + ne], b[:, 2 * r + ne:2 * r + ne + (c - r) // 32]),
                                   codecs.bf16_decode(b[:, :2 * r].copy().view("<u2"))], axis=1)
        return np.concatenate([codecs.e4m3_decode(b[:, :c - r]),
                               codecs.bf16_decode(b[:, c - r:].copy().view("<u2"))], axis=1)
    entries = dec(sc["kv"][0].numpy())
    win = dec(sc["win"][0].numpy())
    qs = synth.queries(cfg, 8, device="cpu", mx_codes=(125, 127))
    q = qs["q"].float().numpy().astype(np.float64)
    ki, qI = cpu_baseline_keys_and_queries(cfg, sc, qs, N) if idx else (None, [None] * 8)
    w = qs["w"].float().numpy().astype(np.float64) if idx else [None] * 8
    h = synth.hidden(cfg, 0, tau, tau + 1, device="cpu").float().numpy().astype(np.float64)
    paths = (("kv_a", "kv_b", "z_a", "z_b", "ki_a", "ki_b", "zi_a", "zi_b") if cfg["dual"]
             else ("kv", "z"))
    n = 0
    t0 = time.perf_counter()
    while True:
        i = n % 8
        for p in paths:
            R.project(h, OW[p])
        _, raw_new, _ = R.raw_rows(h, [tau], OW, od)

        def raw_of(pos, raw_new=raw_new):
            pos = np.asarray(pos)
            return np.where((pos == tau)[:, None], raw_new[0], win[pos % cfg["n_win"]])
        R.query_step(tau, q[i], qI[i], w[i], None, sink, entries, ki, raw_of, N, od)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    what = (f"indexer over {N} entries, top-{cfg['top_k']}, attention over {cfg['top_k']}+{cfg['n_win']} rows"
            if idx else f"dense attention over {N}+{cfg['n_win']} rows")
    if cfg["kv_fmt"] == "q4":
        what += ", MXFP4 main rows"
    return {"value": round(n / el, 2), "unit": "queries/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n} single-query decode steps of the same workload (compress of the new "
                      f"token, {what}{', MXFP4 indexer keys and queries, BF16 scores' if cfg['idx_fmt'] == 'mxfp4' and idx else ''}), "
                      f"synthetic inputs of the same shapes, {el:.1f} s"}


def cpu_baseline_prefill(cfg, seconds):
    """The oracle on a bounded sample of the prefill chunk: the chunk's compression for the
    first 64 tokens plus single-query steps, scaled to tokens/s of the whole chunk's work."""
    import numpy as np

    import synth
    from oracle import codecs
    from oracle import csa_ref as R
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    od = R.Dims(d=cfg["d"], c=cfg["c"], rope_dim=cfg["rope_dim"], n_h=cfg["n_h"], c_I=cfg["c_I"],
                n_hI=cfg["n_hI"], m=cfg["m"], dual=True, top_k=cfg["top_k"], n_win=cfg["n_win"],
                kv_fmt=cfg["kv_fmt"], idx_fmt=cfg["idx_fmt"])
    p0 = cfg["prefix"]
    N = p0 // cfg["m"]
    W = synth.weights(cfg, device="cpu")
    OW = {k: (None if v is None else v.float().numpy().astype(np.float64)) for k, v in W.items()
          if k not in ("gamma_q", "sink")}
    sink = W["sink"].numpy().astype(np.float64)
    sc = synth.synthetic_cache(cfg, 1, N, cfg["n_win"], device="cpu")
    c, r = cfg["c"], cfg["rope_dim"]
    if cfg["kv_fmt"] == "f32":
        entries = sc["kv"][0].numpy().view(np.float32).astype(np.float64)
        win = sc["win"][0].numpy().view(np.float32).astype(np.float64)
    else:
        entries = np.concatenate([codecs.e4m3_decode(sc["kv"][0].numpy()[:, :c - r]),
                                  codecs.bf16_decode(sc["kv"][0].numpy()[:, c - r:].copy().view("<u2"))], 1)
        win = np.concatenate([codecs.e4m3_decode(sc["win"][0].numpy()[:, :c - r]),
                              codecs.bf16_decode(sc["win"][0].numpy()[:, c - r:].copy().view("<u2"))], 1)
    qs = synth.queries(cfg, 8, device="cpu", mx_codes=(125, 127))
    ki, qI = cpu_baseline_keys_and_queries(cfg, sc, qs, N)
    q = qs["q"].float().numpy().astype(np.float64)
    w = qs["w"].float().numpy().astype(np.float64)
    t0 = time.perf_counter()
    H = synth.hidden(cfg, 0, p0, p0 + 64, device="cpu").float().numpy().astype(np.float64)
    R.compress_sequence(H, OW, od)
    t_comp = (time.perf_counter() - t0) / 64
    n = 0
    t1 = time.perf_counter()
    while True:
        i = n % 8
        R.query_step(p0 + i, q[i], qI[i], w[i], None, sink, entries, ki,
                     lambda pos: win[np.asarray(pos) % cfg["n_win"]], N, od)
        n += 1
        if time.perf_counter() - t1 >= seconds:
            break
    t_q = (time.perf_counter() - t1) / n
    return {"value": round(1.0 / (t_comp + t_q), 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"compression of 64 chunk tokens plus {n} single-query steps against the "
                      f"{N}-entry prefix (synthetic inputs of the workload's shapes); per-token cost "
                      f"= compress share + one query"}


# ----------------------------------------------------------------------------- GPU runs


def run_decode(args, cfg):
    import torch

    import long_context_attention_11_amd as L
    import synth

    dev = "cuda:0"
    calibration_copy()
    B, k, m = cfg["B"], cfg["top_k"], cfg["m"]
    has_idx = cfg["top_k"] > 0      # CSA and CSA2 score and select; HCA attends densely
    dims = L.Dims.from_config(cfg)
    W = synth.weights(cfg, device=dev)
    lw = lib_weights(L, W, cfg["dual"])
    N = cfg["prefix"] // m          # entry capacity per sequence
    steps = args.steps or 200
    warm = args.warmup if args.warmup is not None else 10
    # Enough rotating copies that the tensor a launch streams (indexer keys, or the whole cache
    # for the dense variant) is not still held by the 256 MB last-level cache from an earlier
    # step: the set that rotates between two uses of a copy is at least twice that size.
    streamed = B * N * (cfg["c_I"] if has_idx else synth.row_bytes(cfg))
    copies = args.copies or min(16, max(3, -(-2 * MALL_BYTES // streamed) + 1))
    G = copies
    # Step s runs on copy g = s % G at position tau_start + off[g] + s // G: copy g starts off[g]
    # tokens into the open block (taken by untimed one-token steps) and advances one token per
    # cycle.  The offsets spread the copies over the block, so in every cycle about one step in
    # m completes (and stores) an entry, whatever the number of steps.  The prefix stops
    # `room` entries short of the capacity, which leaves room for every entry completed.
    cycles = -(-(warm + steps) // G)
    offs = [(g * m) // G for g in range(G)]
    room = (max(offs) + cycles) // m + 2
    N0 = N - room
    tau_start = m * N0
    tau = tau_start
    t_build = time.perf_counter()
    paged = getattr(args, "paged", False)
    base = build_cache(L, synth, cfg, dims, lw, dev, B, tau_start, N, cfg["n_win"], paged=paged)
    t_build = time.perf_counter() - t_build
    caches = [base] + [clone_cache(base) for _ in range(copies - 1)]

    # per position: the new token of each sequence (its hidden state) and the position
    npos = max(offs) + cycles
    Hc = [torch.stack([synth.hidden(cfg, b, tau_start + c, tau_start + c + 1, device=dev) for b in range(B)])
          for c in range(npos)]
    posc = [torch.full((B,), tau_start + c, dtype=torch.int32, device=dev) for c in range(npos)]
    H1, pos0 = Hc[0], posc[0]
    ws_c = torch.empty(max(1, L.csa_workspace_size(dims, L.OP_COMPRESS, B=B, T=1)), dtype=torch.uint8, device=dev)
    for g, c in enumerate(caches):   # each copy to its starting offset (untimed)
        for j in range(offs[g]):
            L.csa_compress(dims, lw, c, Hc[j], 1, posc[j], ws_c)
    torch.cuda.synchronize()
    qs = synth.queries(cfg, B, device=dev, tag="decode", mx_codes=(125, 127))
    q_seq = torch.arange(B, dtype=torch.int32, device=dev)
    q_pos = torch.full((B,), tau, dtype=torch.int32, device=dev)
    ws_a = torch.empty(max(1, L.csa_workspace_size(dims, L.OP_ATTEND, Q=B, cap=N)), dtype=torch.uint8, device=dev)
    out = torch.empty((B, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device=dev)
    if has_idx:
        ws_t = torch.empty(max(1, L.csa_topk_workspace_size(dims, B, N)), dtype=torch.uint8, device=dev)
        scores = torch.empty((B, N), dtype=torch.bfloat16 if dims.idx_fmt == "mxfp4" else torch.float32,
                             device=dev)
        idx = torch.empty((B, k), dtype=torch.int32, device=dev)

    def k_compress(c):
        L.csa_compress(dims, lw, c, H1, 1, pos0, ws_c)

    def k_index(c):
        L.csa_index_scores(dims, c, qs["qI"], qs["w"], q_seq, q_pos, B, scores, N)

    def k_topk(c):
        L.csa_topk(dims, c, q_seq, q_pos, B, scores, N, idx, ws_t)

    def k_attend(c):
        L.csa_attend(dims, c, qs["q"], W["gamma_q"], W["sink"], q_seq, q_pos, B, idx if has_idx else None, out, ws_a)

    phases = [k_compress, k_index, k_topk, k_attend] if has_idx else [k_compress, k_attend]
    ws_f = torch.empty(max(1, L.csa_workspace_size(dims, L.OP_FORWARD, B=B, T=1, cap=N)), dtype=torch.uint8, device=dev)

    if args.layer:
        # the layer h -> output: query-side projections, the path, grouped output projection
        PW = synth.proj_weights(cfg, cfg["d_c"], cfg["g"], cfg["d_g"], device=dev)
        pw = L.ProjWeights(**PW)
        h = H1.reshape(B, cfg["d"])
        q_l = torch.empty_like(qs["q"])
        qI_l = torch.empty_like(qs["qI"]) if has_idx else None
        w_l = torch.empty_like(qs["w"]) if has_idx else None
        y = torch.empty((B, cfg["d"]), dtype=torch.bfloat16, device=dev)
        ws_q = torch.empty(max(1, L.csa_query_project_workspace_size(dims, pw, B)), dtype=torch.uint8, device=dev)
        ws_o = torch.empty(max(1, L.csa_output_project_workspace_size(dims, pw, B)), dtype=torch.uint8, device=dev)

        def k_qproj(c):
            L.csa_query_project(dims, pw, h, B, q_l, qI_l, w_l, ws_q)

        def k_oproj(c):
            L.csa_output_project(dims, pw, out, B, y, ws_o)

    def step(s):
        # step s: one pass of the whole path through the library's forward entry point, on
        # copy s % G at position tau_start + off[s % G] + s // G
        c, cyc = caches[s % G], offs[s % G] + s // G
        if args.layer:
            k_qproj(c)
            L.csa_forward(dims, lw, c, Hc[cyc], 1, posc[cyc], q_l, qI_l, w_l, W["gamma_q"], W["sink"], out,
                          idx if has_idx else None, ws_f)
            k_oproj(c)
            return
        L.csa_forward(dims, lw, c, Hc[cyc], 1, posc[cyc], qs["q"], qs["qI"] if has_idx else None,
                      qs["w"] if has_idx else None, W["gamma_q"], W["sink"], out,
                      idx if has_idx else None, ws_f)

    def graphs(s0, s1):
        # steps s0 .. s1 - 1 in graphs of at most one cycle each (a decode loop over the copies
        # captured once per cycle), cut at cycle boundaries
        gs, s = [], s0
        while s < s1:
            e = min(s1, (s // G + 1) * G)
            gs.append(capture(lambda s=s, e=e: [step(i) for i in range(s, e)]))
            s = e
        return gs

    g_warm, g_timed = graphs(0, warm), graphs(warm, warm + steps)
    torch.cuda.synchronize()
    for g in g_warm:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for g in g_timed:
        g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the last step again, eagerly: a step at a position a copy has already taken recomputes
    # exactly what it wrote then, so the graph's output must be reproduced bit for bit
    got = (y.clone() if args.layer else out.clone(), idx.clone() if has_idx else None)
    step(warm + steps - 1)
    torch.cuda.synchronize()
    ok = torch.equal(y if args.layer else out, got[0]) and (not has_idx or torch.equal(idx, got[1]))

    # per-kernel launch durations (same inputs and grids, rotating cache copies)
    kt = {name: kernel_time_us([lambda c=c, f=f: f(c) for c in caches])
          for name, f in zip(["compress", "index_scores", "topk", "attend"] if has_idx else ["compress", "attend"], phases)}
    if has_idx:
        # scoring and selection in one call: the indexer, the threshold pass and the final
        # selection, the same kernels as in the step but without the projection and the fold
        ws_it = torch.empty(max(1, L.csa_workspace_size(dims, L.OP_INDEX_TOPK, Q=B, cap=N)), dtype=torch.uint8,
                            device=dev)
        kt["index_topk"] = kernel_time_us([lambda c=c: L.csa_index_topk(dims, c, qs["qI"], qs["w"], q_seq, q_pos, B,
                                                                         idx, None, ws_it) for c in caches])
        del ws_it
    if args.layer:
        kt["q_proj"] = kernel_time_us([lambda c=c: k_qproj(c) for c in caches])
        kt["o_proj"] = kernel_time_us([lambda c=c: k_oproj(c) for c in caches])
    res = {
        "metric": ("CSA decode queries/s (Flash-shaped, 128K context, batch 16)"
                   if cfg["name"] == "c2" and not args.layer and not paged
                   else f"CSA {'attention-layer ' if args.layer else ''}decode queries/s ({cfg['name']}"
                        f"{', paged cache' if paged else ''})"),
        "value": round(B * steps / wall, 1), "unit": "queries/s", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": round(wall / steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": (("MXFP4 MFMA indexer, bf16 index scores; " if cfg["idx_fmt"] == "mxfp4" else "")
                  + ("bf16 MFMA on MXFP4/bf16 KV storage" if cfg["kv_fmt"] == "q4" else "bf16 MFMA on E4M3/bf16 KV storage")
                  + ", fp32 accumulate"),
        "data": "synthetic (seeded N(0,1) hidden states and queries, N(0,1/fan_in) weights)",
    }
    if has_idx:
        key_bytes = cfg["c_I"] // 2 + cfg["c_I"] // 32 if cfg["idx_fmt"] == "mxfp4" else cfg["c_I"]
        bytes_per_query = N * key_bytes + cfg["n_hI"] * key_bytes + 2 * cfg["n_hI"]
        alg = B * bytes_per_query
        dur = kt["index_scores"] * 1e-6
        kname = "k_indexer_fp4" if cfg["idx_fmt"] == "mxfp4" else "k_indexer_bf16"
        res["roofline"] = {"bound": "hbm", "kernel": f"indexer ({kname})",
                           "achieved": round(alg / dur / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                           "frac": round(alg / dur / HBM_PEAK, 4),
                           "traffic": measured_traffic() if cfg["name"] == "c2" and not paged else None,
                           "alg_bytes_per_launch": alg, "avg_launch_us": round(kt["index_scores"], 2),
                           "with_selection": {"call": "csa_index_topk", "avg_us": round(kt["index_topk"], 2),
                                              "frac_including_selection": round(alg / (kt["index_topk"] * 1e-6) / HBM_PEAK, 4)}}
    else:
        rows = N + cfg["n_win"]
        alg = B * (rows * 576 + 2 * 2 * cfg["n_h"] * cfg["c"])
        dur = kt["attend"] * 1e-6
        res["roofline"] = {"bound": "hbm", "kernel": "attention (k_attend_hs + combine)",
                           "achieved": round(alg / dur / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                           "frac": round(alg / dur / HBM_PEAK, 4), "traffic": None,
                           "alg_bytes_per_launch": alg, "avg_launch_us": round(kt["attend"], 2)}
    if has_idx:
        rows = k + cfg["n_win"]
        at_bytes = B * (rows * synth_row_bytes(cfg) + 2 * 2 * cfg["n_h"] * cfg["c"] + 4 * k)
        at_flops = B * 2.0 * 2.0 * cfg["n_h"] * cfg["c"] * rows
        t_at = kt["attend"] * 1e-6
        res["roofline_attention"] = {
            "bound": "hbm", "kernel": "attention (csa_attend: k_attend_hs + combine)",
            "achieved": round(at_bytes / t_at / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": round(at_bytes / t_at / HBM_PEAK, 4), "alg_bytes_per_launch": at_bytes,
            "mfma_frac": round(at_flops / t_at / BF16_PEAK, 4), "avg_launch_us": round(kt["attend"], 2)}
    res["kernels_us"] = {k_: round(v, 2) for k_, v in kt.items()}
    res["graph_replay_matches_eager"] = bool(ok)
    res["cache_build_s"] = round(t_build, 2)
    desc = {"c2": "Flash-shaped CSA decode, 16 seqs x 131072-token context (32768 entries), d=4096, "
                  "64 heads x 512, indexer 64x128, top-k 512, n_win 128, one new token per sequence per step",
            "c2fp4": "Flash-shaped CSA decode as c2, with the indexer's keys and queries in MXFP4 "
                     "(the pages' FP4 indexer path)",
            "c3": "Pro-shaped CSA decode, 4 seqs x 1048576-token context (262144 entries), d=7168, "
                  "128 heads x 512, indexer 64x128, top-k 1024, n_win 128",
            "c5": "HCA decode, 8 seqs x 1048576-token context (8192 entries, m'=128), d=4096, "
                  "64 heads x 512, dense, n_win 128",
            "c6": "CSA2 decode (single-path fold with m=4 and no bias, index keys projected from the "
                  "entry, MXFP4 main KV rows of 384 B), 16 seqs x 131072-token context (32768 entries), "
                  "d=4096, 64 heads x 512, indexer 64x128, top-k 512, n_win 128",
            "c6fp4": "CSA2 decode as c6, with the indexer's keys and queries in MXFP4"}[cfg["name"]]
    if paged:
        desc += (f"; paged cache: {PAGE_TOKENS}-token pages ({PAGE_TOKENS // m} entries) dealt over a shuffled "
                 f"pool through a per-sequence block table")
    if args.layer:
        # the projections stream their weights once per step: HBM-bound at decode
        d, dc, nq = cfg["d"], cfg["d_c"], cfg["n_h"] * cfg["c"]
        wq = 2 * (dc * d + nq * dc + ((cfg["n_hI"] * cfg["c_I"] * dc + cfg["n_hI"] * d) if has_idx else 0))
        wo = 2 * (nq * cfg["d_g"] + d * cfg["g"] * cfg["d_g"])
        tq, to = kt["q_proj"] * 1e-6, kt["o_proj"] * 1e-6
        res["roofline_projections"] = {
            "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK / 1e9,
            "query_side": {"weight_bytes": wq, "us": round(kt["q_proj"], 2), "achieved": round(wq / tq / 1e9, 1),
                           "frac": round(wq / tq / HBM_PEAK, 4)},
            "output_side": {"weight_bytes": wo, "us": round(kt["o_proj"], 2), "achieved": round(wo / to / 1e9, 1),
                            "frac": round(wo / to / HBM_PEAK, 4)}}
        desc += (f"; whole attention layer: query-side projections (d_c {cfg['d_c']}) before the path and the "
                 f"grouped output projection (g {cfg['g']}, d_g {cfg['d_g']}) after it")
    res["config"] = {"workload": f"{cfg['name']}: {desc}", "global_batch": B, "seq_len": cfg["prefix"],
                     "positions": f"{tau_start} .. {tau_start + npos - 1} (copy g starts {offs} tokens into the "
                                  f"open block and advances one token per cycle; about one step in {m} completes "
                                  f"an entry)",
                     "parallelism": "single GPU", "launch": f"HIP graphs of {G} steps (one per cache copy)",
                     "cache_copies": G}
    if not args.no_cpu and not args.layer:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    return res, ok


def prefill_rooflines(L, cfg, dims, cache, qs, W, idx, out, p0, T, q_chunk, ws):
    """The chunk's dominant kernels timed on their own with the forward's grids: the indexer
    on its first q_chunk queries (the forward runs it chunk by chunk, as csa_index_scores_grouped
    does), and the attention over all T queries with the forward's selection."""
    import torch
    m, cap = cfg["m"], cache.cap
    Qc = q_chunk
    fp4 = cfg["idx_fmt"] == "mxfp4"
    q_seq = torch.zeros(Qc, dtype=torch.int32, device="cuda")
    q_pos = torch.arange(p0, p0 + Qc, dtype=torch.int32, device="cuda")
    scores = torch.empty((Qc, cap), dtype=torch.bfloat16 if fp4 else torch.float32, device="cuda")
    qI = qs["qI"][:Qc].contiguous()
    wI = qs["w"][:Qc].contiguous()
    t_scores = kernel_time_us([lambda: L.csa_index_scores_grouped(dims, cache, qI, wI, q_seq, q_pos, Qc, scores, cap)],
                              reps=5, rounds=3)
    del scores
    flops = 2.0 * cfg["n_hI"] * cfg["c_I"] * sum(min((p0 + t) // m, cap) for t in range(Qc))
    peak = FP4_PEAK if fp4 else BF16_PEAK
    if fp4:
        t_ix, kname = t_scores, "k_indexer_tile_fp4"
    else:
        # the forward's own path: the indexer that thresholds its scores, then the selection
        # from its lists (the launch pair csa_index_topk_grouped makes; the selection is ~1 %)
        idx_c = torch.empty((Qc, cfg["top_k"]), dtype=torch.int32, device="cuda")
        t_ix = kernel_time_us([lambda: L.csa_index_topk_grouped(dims, cache, qI, wI, q_seq, q_pos, Qc, idx_c, None, ws)],
                              reps=5, rounds=3)
        kname = "k_indexer_tile<true> (own threshold) + k_topk_final"
        del idx_c
    ix = {"bound": "mfma", "kernel": kname, "queries_per_launch": Qc,
          "achieved": round(flops / (t_ix * 1e-6) / 1e12, 1), "peak": peak / 1e12, "unit": "TFLOP/s",
          "frac": round(flops / (t_ix * 1e-6) / peak, 4), "traffic": None,
          "alg_flop_per_launch": flops, "avg_launch_us": round(t_ix, 1), "scores_only_kernel_us": round(t_scores, 1),
          "contraction": "MXFP4 block-scaled MFMA" if fp4 else "bf16 MFMA on E4M3 widened exactly (fp8 MFMA inexact)"}
    if not fp4:
        ix["frac_of_fp8_peak"] = round(flops / (t_ix * 1e-6) / FP8_PEAK, 4)
    q_seq_all = torch.zeros(T, dtype=torch.int32, device="cuda")
    q_pos_all = torch.arange(p0, p0 + T, dtype=torch.int32, device="cuda")
    # (the forward's workspace holds the sparse attention's partials)
    t_at = kernel_time_us([lambda: L.csa_attend(dims, cache, qs["q"], W["gamma_q"], W["sink"], q_seq_all, q_pos_all,
                                                T, idx, out, ws)], reps=5, rounds=3)
    rows = cfg["top_k"] + cfg["n_win"]
    at_bytes = T * (rows * synth_row_bytes(cfg) + 2 * 2 * cfg["n_h"] * cfg["c"] + 4 * cfg["top_k"])
    at_flops = T * 2.0 * 2.0 * cfg["n_h"] * cfg["c"] * rows
    at = {"bound": "mfma", "kernel": "k_attend_hs (prefill)", "achieved": round(at_flops / (t_at * 1e-6) / 1e12, 1),
          "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s", "frac": round(at_flops / (t_at * 1e-6) / BF16_PEAK, 4),
          "alg_flop_per_launch": at_flops, "alg_bytes_per_launch": at_bytes,
          "hbm_frac_without_reuse": round(at_bytes / (t_at * 1e-6) / HBM_PEAK, 4), "avg_launch_us": round(t_at, 1)}
    return {"roofline": ix, "roofline_attention": at}


def synth_row_bytes(cfg):
    import synth
    return synth.row_bytes(cfg)


def run_prefill(args, cfg):
    import torch

    import long_context_attention_11_amd as L
    import synth

    dev = "cuda:0"
    T, p0, k = cfg["T"], cfg["prefix"], cfg["top_k"]
    dims = L.Dims.from_config(cfg)
    W = synth.weights(cfg, device=dev)
    lw = lib_weights(L, W, True)
    cap = (p0 + T) // cfg["m"]
    win_cap = T + cfg["n_win"]
    t_build = time.perf_counter()
    cache = build_cache(L, synth, cfg, dims, lw, dev, 1, p0, cap, win_cap) if p0 else \
        L.Cache(dims, B=1, cap=cap, win_cap=win_cap, device=dev)
    t_build = time.perf_counter() - t_build
    H = synth.hidden(cfg, 0, p0, p0 + T, device=dev).unsqueeze(0).contiguous()
    qs = synth.queries(cfg, T, device=dev, tag="prefill", mx_codes=(125, 127))
    pos0 = torch.full((1,), p0, dtype=torch.int32, device=dev)
    dt = torch.float32 if cfg["act"] == "f32" else torch.bfloat16
    out = torch.empty((T, cfg["n_h"], cfg["c"]), dtype=dt, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    q_chunk = min(T, 4096)
    ws = torch.empty(L.csa_workspace_size(dims, L.OP_FORWARD, B=1, T=T, cap=cap, q_chunk=q_chunk),
                     dtype=torch.uint8, device=dev)

    if args.layer:
        # the layer h -> output for the chunk: query-side projections, the path, grouped output
        PW = synth.proj_weights(cfg, cfg["d_c"], cfg["g"], cfg["d_g"], device=dev)
        pw = L.ProjWeights(**PW)
        h2 = H.reshape(T, cfg["d"])
        q_l, qI_l, w_l = torch.empty_like(qs["q"]), torch.empty_like(qs["qI"]), torch.empty_like(qs["w"])
        y = torch.empty((T, cfg["d"]), dtype=torch.bfloat16, device=dev)
        ws_q = torch.empty(max(1, L.csa_query_project_workspace_size(dims, pw, T)), dtype=torch.uint8, device=dev)
        ws_o = torch.empty(max(1, L.csa_output_project_workspace_size(dims, pw, T)), dtype=torch.uint8, device=dev)

    def step():
        if args.layer:
            L.csa_query_project(dims, pw, h2, T, q_l, qI_l, w_l, ws_q)
            L.csa_forward(dims, lw, cache, H, T, pos0, q_l, qI_l, w_l, W["gamma_q"], W["sink"], out, idx, ws)
            L.csa_output_project(dims, pw, out, T, y, ws_o)
            return
        L.csa_forward(dims, lw, cache, H, T, pos0, qs["q"], qs["qI"], qs["w"], W["gamma_q"], W["sink"],
                      out, idx, ws)

    step()
    torch.cuda.synchronize()
    steps = args.steps or (5 if p0 else 50)
    warm = args.warmup if args.warmup is not None else 1
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(steps):
        step()
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev[0].elapsed_time(ev[1]) / steps
    res = {"metric": f"CSA {'attention-layer ' if args.layer else ''}prefill tokens/s ({cfg['name']})",
           "value": round(T * steps / wall, 1),
           "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm,
           "ms_per_step": round(wall / steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None,
           "dtype": ("fp32" if cfg["act"] == "f32" else
                     "MXFP4 MFMA indexer, bf16 index scores; bf16 MFMA on E4M3/bf16 KV storage, fp32 accumulate"
                     if cfg["idx_fmt"] == "mxfp4" else "bf16 MFMA on E4M3/bf16 storage, fp32 accumulate"),
           "data": "synthetic (seeded N(0,1) hidden states and queries, N(0,1/fan_in) weights)",
           "gpu_ms_per_step": round(gpu_ms, 4), "cache_build_s": round(t_build, 2),
           "config": {"workload": f"{cfg['name']}: chunked prefill, {T}-token chunk after a {p0}-token prefix, "
                                  f"d={cfg['d']}, {cfg['n_h']} heads x {cfg['c']}, top-k {k}",
                      "global_batch": 1, "seq_len": p0 + T, "parallelism": "single GPU",
                      "launch": "eager csa_forward"}}
    if cfg["kv_fmt"] != "f32":
        # the indexer's contraction: per query 64 heads x 128 dims x V entries, 2 FLOP each
        Vs = [min((p0 + t) // cfg["m"], cap) for t in range(T)]
        flops = 2.0 * cfg["n_hI"] * cfg["c_I"] * sum(Vs)
        res["indexer_tflop_per_step"] = round(flops / 1e12, 2)
        if not args.layer:
            res.update(prefill_rooflines(L, cfg, dims, cache, qs, W, idx, out, p0, T, q_chunk, ws))
    if args.layer:
        d, dc, nq = cfg["d"], cfg["d_c"], cfg["n_h"] * cfg["c"]
        res["projection_tflop_per_step"] = round(2.0 * T * (d * (dc + cfg["n_hI"]) + dc * (nq + cfg["n_hI"] * cfg["c_I"])
                                                          + nq * cfg["d_g"] + cfg["g"] * cfg["d_g"] * d) / 1e12, 2)
        res["config"]["workload"] += (f"; whole attention layer: query-side projections (d_c {cfg['d_c']}) and the "
                                      f"grouped output projection (g {cfg['g']}, d_g {cfg['d_g']})")
    if not args.no_cpu and cfg["name"] != "c1" and not args.layer:
        res["cpu_baseline"] = cpu_baseline_prefill(cfg, args.cpu_seconds)
    return res, True


def attention_batch_series(cfg, batches=(16, 32, 64, 128, 256), reps=20):
    """Decode attention (csa_attend, the launches the step runs) at the Flash shape for B
    queries, each over its own sequence: 512 selected entries drawn at random (a fresh draw
    per launch) plus the 128-row window.  Caches large enough (capacity up to 262144 entries
    per sequence, at most ~20 GB) that the rows a launch gathers were not fetched by the
    launches just before it, so the bytes come from HBM.  Shows where the latency floor of a
    small batch gives way to the bandwidth bound."""
    import torch

    import long_context_attention_11_amd as L
    import synth
    dims = L.Dims.from_config(cfg)
    k, nw, rb = cfg["top_k"], cfg["n_win"], synth_row_bytes(cfg)
    r = cfg["c"] - cfg["rope_dim"]
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    out_rows = []
    for B in batches:
        cap = max(4096, min(262144, (20 << 30) // (B * rb)))
        cache = L.Cache(dims, B=B, cap=cap, win_cap=nw, device="cuda")
        for t in (cache.kv, cache.win):
            t.copy_(torch.randint(0, 0x60, tuple(t.shape), generator=g, device="cuda", dtype=torch.uint8))
            t.view(t.shape[0], t.shape[1], rb)[:, :, r + 1::2] = 0x3F   # bf16 RoPE dims of magnitude ~1
        tau = 4 * cap
        cache.n_entries.fill_(cap)
        cache.win_pos.copy_(torch.arange(tau - nw + 1, tau + 1, dtype=torch.int32, device="cuda")
                            .roll((tau + 1) % nw).repeat(B, 1))
        qs = synth.queries(cfg, B, device="cuda", tag="series")
        W = {"gamma_q": torch.ones(cfg["c"], device="cuda"),
             "sink": synth.randn((cfg["n_h"],), 0.1 ** 0.5, "cuda", 0, "sink")}
        q_seq = torch.arange(B, dtype=torch.int32, device="cuda")
        q_pos = torch.full((B,), tau, dtype=torch.int32, device="cuda")
        idxs = [torch.sort(torch.randint(0, cap, (B, k), generator=g, device="cuda", dtype=torch.int32), 1).values
                for _ in range(reps)]
        out = torch.empty((B, cfg["n_h"], cfg["c"]), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(1, L.csa_workspace_size(dims, L.OP_ATTEND, Q=B, cap=cap)), dtype=torch.uint8, device="cuda")
        us = kernel_time_us([lambda i=i: L.csa_attend(dims, cache, qs["q"], W["gamma_q"], W["sink"], q_seq, q_pos, B,
                                                      idxs[i], out, ws) for i in range(reps)], reps=reps)
        byt = B * ((k + nw) * rb + 2 * 2 * cfg["n_h"] * cfg["c"] + 4 * k)
        out_rows.append({"B": B, "us": round(us, 2), "alg_bytes": byt, "GB_s": round(byt / us / 1e3, 1),
                         "frac_hbm": round(byt / (us * 1e-6) / HBM_PEAK, 4), "cache_entries_per_seq": cap})
        del cache, idxs, out, ws
        torch.cuda.empty_cache()
    return out_rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    torch.cuda.set_device(0)
    cfg = synth.config(args.config)
    if args.config in ("c2", "c2fp4", "c3", "c5", "c6", "c6fp4"):
        res, ok = run_decode(args, cfg)
    else:
        res, ok = run_prefill(args, cfg)
    if args.config == "c2" and not args.layer and not args.no_extra:
        # the rest of the metric in the same run: decode at 1M context (Pro shape), prefill
        # tokens/s after a 1M-token prefix, and the decode attention's batch series
        print(f"[bench] c2 done ({res['value']} queries/s); c3 decode", file=sys.stderr, flush=True)
        extra = {}
        sub = argparse.Namespace(**{**vars(args), "steps": 20, "warmup": 5, "no_cpu": True, "copies": None})
        r3, ok3 = run_decode(sub, synth.config("c3"))
        extra["c3_decode"] = {k_: r3[k_] for k_ in ("metric", "value", "unit", "ms_per_step", "roofline",
                                                    "roofline_attention", "kernels_us", "graph_replay_matches_eager")}
        extra["c3_decode"]["workload"] = r3["config"]["workload"]
        print(f"[bench] c3 done ({r3['value']} queries/s); c2 decode on a paged cache", file=sys.stderr, flush=True)
        sub = argparse.Namespace(**{**vars(args), "steps": 20, "warmup": 5, "no_cpu": True, "copies": None,
                                    "paged": True})
        rp, okp = run_decode(sub, cfg)
        extra["c2_decode_paged"] = {k_: rp[k_] for k_ in ("metric", "value", "unit", "ms_per_step", "roofline",
                                                          "roofline_attention", "kernels_us",
                                                          "graph_replay_matches_eager")}
        extra["c2_decode_paged"]["workload"] = rp["config"]["workload"]
        ok3 = ok3 and okp
        print(f"[bench] paged c2 done ({rp['value']} queries/s); c6 (CSA2) decode", file=sys.stderr, flush=True)
        sub = argparse.Namespace(**{**vars(args), "steps": 20, "warmup": 5, "no_cpu": True, "copies": None,
                                    "paged": False})
        r6, ok6 = run_decode(sub, synth.config("c6"))
        extra["c6_decode"] = {k_: r6[k_] for k_ in ("metric", "value", "unit", "ms_per_step", "roofline",
                                                    "roofline_attention", "kernels_us", "graph_replay_matches_eager")}
        extra["c6_decode"]["workload"] = r6["config"]["workload"]
        ok3 = ok3 and ok6
        print(f"[bench] c6 done ({r6['value']} queries/s); c4a prefill", file=sys.stderr, flush=True)
        sub = argparse.Namespace(**{**vars(args), "steps": 3, "warmup": 1, "no_cpu": True})
        r4, _ = run_prefill(sub, synth.config("c4a"))
        extra["c4a_prefill"] = {k_: r4[k_] for k_ in ("metric", "value", "unit", "ms_per_step", "roofline",
                                                      "roofline_attention", "indexer_tflop_per_step")}
        extra["c4a_prefill"]["workload"] = r4["config"]["workload"]
        print(f"[bench] c4a done ({r4['value']} tokens/s); attention batch series", file=sys.stderr, flush=True)
        extra["decode_attention_batch_series"] = attention_batch_series(synth.config("c2"))
        res["extra"] = extra
        ok = ok and ok3
    print(json.dumps(res), flush=True)
    if not ok:
        sys.exit(1)


if __name__ == "__main__":
    main()
