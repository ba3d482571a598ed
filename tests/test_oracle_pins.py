"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU needed).

Each test checks the oracle against something other than itself: a figure or worked example
the pages print (tests/golden/), a closed form, an invariant, brute force on a tiny input,
exact rational arithmetic, or a library routine (torch casts, torch SDPA in float64).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs
from oracle import csa_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dims(**kw):
    base = dict(d=32, c=16, rope_dim=8, n_h=3, c_I=8, n_hI=2, m=4, dual=True, top_k=4, n_win=4)
    base.update(kw)
    return R.Dims(**base)


def _weights(dims, rng, dtype=np.float64):
    d, c, cI, m = dims.d, dims.c, dims.c_I, dims.m
    W = {}
    if dims.dual:
        for nm in ("kv_a", "kv_b", "z_a", "z_b"):
            W[nm] = rng.standard_normal((c, d)) / math.sqrt(d)
        for nm in ("ki_a", "ki_b", "zi_a", "zi_b"):
            W[nm] = rng.standard_normal((cI, d)) / math.sqrt(d)
        W["B_a"] = rng.standard_normal((m, c)) * 0.3
        W["B_b"] = rng.standard_normal((m, c)) * 0.3
        W["BI_a"] = rng.standard_normal((m, cI)) * 0.3
        W["BI_b"] = rng.standard_normal((m, cI)) * 0.3
    else:
        W["kv"] = rng.standard_normal((c, d)) / math.sqrt(d)
        W["z"] = rng.standard_normal((c, d)) / math.sqrt(d)
        W["B"] = rng.standard_normal((m, c)) * 0.3
    W["gamma_kv"] = None
    return W


# ----------------------------------------------------------------------------- codecs


def test_e4m3_table_matches_format_definition():
    v = codecs.e4m3_values()
    # Hand-derived from the OCP E4M3 bit layout (bias 7, 3 mantissa bits, no infinities).
    assert v[0x00] == 0.0
    assert v[0x01] == 2.0 ** -9  # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9  # largest subnormal
    assert v[0x08] == 2.0 ** -6  # smallest normal
    assert v[0x38] == 1.0
    assert v[0x39] == 1.125
    assert v[0x7E] == 448.0  # largest finite
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    assert v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) == -1.0
    assert v[0xFE] == -448.0
    # 126 distinct positive finite values plus zero
    pos = v[:0x7F]
    assert len(set(pos.tolist())) == 127


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = codecs.e4m3_decode(codes)
    both_nan = np.isnan(t) & np.isnan(mine)
    assert np.all(both_nan | (t == mine))


def test_e4m3_encode_round_trip_and_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 3, rng.uniform(-448, 448, 20000),
                        rng.standard_normal(5000) * 0.01])
    x = codecs.to_f32(x)
    mine = codecs.e4m3_encode(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of values that round to zero as well; compare decoded values, and
    # codes where the value is non-zero
    assert np.array_equal(codecs.e4m3_decode(mine), codecs.e4m3_decode(ref))
    # every code decodes to itself
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(codecs.e4m3_encode(codecs.e4m3_decode(codes)), codes)


def test_e4m3_ties_to_even_and_saturation():
    enc = codecs.e4m3_encode
    assert enc(1.0625)[()] == 0x38  # midway 1.0 (0x38, even) / 1.125 (0x39)
    assert enc(1.1875)[()] == 0x3A  # midway 1.125 (0x39) / 1.25 (0x3a, even)
    assert enc(2.0 ** -10)[()] == 0x00  # half the smallest subnormal -> even code 0
    assert enc(3 * 2.0 ** -10)[()] == 0x02  # midway 1 and 2 subnormal units -> 2 (even)
    assert enc(449.0)[()] == 0x7E and enc(1e9)[()] == 0x7E and enc(-1e9)[()] == 0xFE
    assert enc(464.0)[()] == 0x7E  # past the 448/480 midpoint still saturates
    assert enc(float("nan"))[()] == 0x7F
    assert enc(-0.0)[()] == 0x80 and enc(-(2.0 ** -11))[()] == 0x80


def test_bf16_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(50000) * 10, rng.standard_normal(1000) * 1e-30])
    x32 = x.astype(np.float32)
    # add exact ties: float32 values whose low 16 bits are 0x8000
    ties = (rng.integers(0, 2 ** 15, 2000).astype(np.uint32) << 16 | 0x8000).astype(np.uint32)
    ties |= np.uint32(0x3F000000) & np.uint32(0x7F800000)
    x32 = np.concatenate([x32, ties.view(np.float32)])
    x32 = x32[np.isfinite(x32)]
    mine = codecs.bf16_encode(x32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(codecs.bf16_decode(mine), torch.from_numpy(x32).to(torch.bfloat16).double().numpy())


# ----------------------------------------------------------------------------- fold


def test_e2m1_e8m0_tables_match_format_definition():
    """OCP MX v1.0: E2M1 positive values 0, 0.5, 1, 1.5, 2, 3, 4, 6 (code 8 is -0); E8M0
    code c is 2^(c - 127), 255 is NaN.  Values written out by hand, not by the oracle's
    formula."""
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    t = codecs.e2m1_values()
    assert list(t[:8]) == pos
    assert list(-t[8:]) == pos and np.signbit(t[8])
    assert codecs.e8m0_decode(127) == 1.0 and codecs.e8m0_decode(128) == 2.0
    assert codecs.e8m0_decode(0) == 2.0 ** -127 and codecs.e8m0_decode(254) == 2.0 ** 127
    assert np.isnan(codecs.e8m0_decode(255))


def test_mxfp4_rounding_ties_and_saturation():
    """Scaled values at every midpoint round to the even code; past 6 they saturate."""
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    assert list(codecs.e2m1_decode(codecs.e2m1_encode_scaled(ties, 0))) == want
    assert list(codecs.e2m1_decode(codecs.e2m1_encode_scaled(-ties, 0))) == [-v for v in want]
    near = np.array([0.26, 0.74, 1.26, 1.74, 2.51, 3.49, 5.01, 6.5, 7.99, 100.0])
    assert list(codecs.e2m1_decode(codecs.e2m1_encode_scaled(near, 0))) == \
        [0.5, 0.5, 1.5, 1.5, 3.0, 3.0, 6.0, 6.0, 6.0, 6.0]
    # the same decisions at another scale: X = 2^-3
    assert list(codecs.e2m1_decode(codecs.e2m1_encode_scaled(ties / 8, -3))) == want
    # brute force: the chosen magnitude is the nearest, ties to the even code
    rng = np.random.default_rng(7)
    a = rng.uniform(0, 6, 20000)
    got = codecs.e2m1_encode_scaled(a, 0) & 7
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    for x, g in zip(a.astype(np.float32).astype(np.float64), got):
        d = np.abs(mags - x)
        best = np.flatnonzero(d == d.min())
        assert g == (best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0])


def test_mxfp4_scale_rule_and_round_trip():
    """X = 2^(floor(log2 max|v|) - 2) per block of 32; representable blocks come back
    unchanged; blocks are independent; an all-zero block takes X = 1."""
    blk = np.zeros((1, 32)); blk[0, 3] = 1.0                     # max 1 -> X = 2^-2, 1/X = 4
    c, s = codecs.mxfp4_encode(blk)
    assert s[0, 0] == 127 - 2 and codecs.e2m1_decode(c[0, 3]) == 4.0
    for amax, e in ((4.0, 0), (7.99, 0), (8.0, 1), (0.3, -4), (6.0 * 2.0 ** -10, -10)):
        b = np.zeros((1, 32)); b[0, 0] = amax
        assert codecs.mxfp4_scale_exponent(b)[0, 0] == e, (amax, e)
    z = np.zeros((2, 64))
    c, s = codecs.mxfp4_encode(z)
    assert np.all(s == 127) and np.all(c == 0)
    rng = np.random.default_rng(3)
    vals = codecs.e2m1_values()[rng.integers(0, 16, (50, 64))]
    vals[:, 0], vals[:, 32] = 6.0, -4.0                          # each block's max is 4 or 6
    scale = np.ldexp(1.0, rng.integers(-6, 4, (50, 2)))
    x = vals * np.repeat(scale, 32, axis=1)
    c, s = codecs.mxfp4_encode(x)
    assert np.array_equal(codecs.mxfp4_decode(codecs.mxfp4_pack(c), s), x)
    c1, s1 = codecs.mxfp4_encode(x[:, :32])
    c2, s2 = codecs.mxfp4_encode(x[:, 32:])
    assert np.array_equal(c, np.concatenate([c1, c2], 1)) and np.array_equal(s, np.concatenate([s1, s2], 1))
    assert codecs.mxfp4_pack(np.array([1, 2], np.uint8))[0] == 0x21
    assert np.array_equal(codecs.mxfp4_unpack(np.array([0x9F], np.uint8)), [0xF, 0x9])


def test_bf16_round_nearest_exact():
    """Rounding straight from float64: ties to even, and a value just above a tie rounds up
    where a float32 step would first land on the tie (the double-rounding case); random
    values agree with an exact nearest search over the neighbouring bfloat16 values."""
    ulp = 2.0 ** -7
    cases = [(1.0 + ulp / 2, 1.0), (1.0 + 3 * ulp / 2, 1.0 + 2 * ulp), (-(1.0 + ulp / 2), -1.0),
             (1.0 + ulp / 2 + 2.0 ** -30, 1.0 + ulp), (3.0, 3.0), (0.0, 0.0)]
    for x, want in cases:
        assert codecs.bf16_round_nearest(x) == want, (x, want)
    rng = np.random.default_rng(21)
    xs = rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000))
    got = codecs.bf16_round_nearest(xs)
    for x, g in zip(xs, got):
        f, e = math.frexp(x)
        lo = math.floor(f * 256) / 256 * 2.0 ** e
        hi = lo + 2.0 ** (e - 8)
        dl, dh = Fraction(x) - Fraction(lo), Fraction(hi) - Fraction(x)
        if dl < dh:
            want = lo
        elif dh < dl:
            want = hi
        else:
            want = lo if int(abs(lo) / 2.0 ** (e - 8)) % 2 == 0 else hi
        assert g == want, (x, g, want)
        # the result is a bfloat16 value
        assert codecs.bf16_decode(codecs.bf16_encode(g)) == g


def test_fold_softmax_columns_sum_to_one():
    rng = np.random.default_rng(3)
    n, c, m = 24, 7, 4
    A = [rng.standard_normal((n, c)) for _ in range(4)]
    Ba, Bb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
    _, S = R.csa_fold(*A, Ba, Bb, m, return_weights=True)
    assert S.shape == (n // m, 2 * m, c)
    assert np.allclose(S.sum(axis=1), 1.0, atol=1e-12, rtol=0)
    assert np.all(S[0, m:] == 0.0)  # entry 0: b half has weight 0
    _, S2 = R.hca_fold(A[0], A[1], rng.standard_normal((m, c)), m, return_weights=True)
    assert np.allclose(S2.sum(axis=1), 1.0, atol=1e-12, rtol=0)


def test_fold_closed_forms():
    rng = np.random.default_rng(4)
    n, c, m = 20, 5, 4
    v = rng.standard_normal(c)
    const = np.tile(v, (n, 1))
    Za, Zb = rng.standard_normal((n, c)) * 3, rng.standard_normal((n, c)) * 3
    Ba, Bb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
    # constant rows: any convex combination returns the constant
    out = R.csa_fold(const, const, Za, Zb, Ba, Bb, m)
    assert np.allclose(out, v, atol=1e-12)
    # zero logits and biases: plain mean of the 2m rows (m rows for entry 0)
    Ca, Cb = rng.standard_normal((n, c)), rng.standard_normal((n, c))
    z = np.zeros((n, c))
    zb = np.zeros((m, c))
    out = R.csa_fold(Ca, Cb, z, z, zb, zb, m)
    assert np.allclose(out[0], Ca[0:4].mean(0), atol=1e-12)
    for i in range(1, n // m):
        ref = (Ca[m * i:m * (i + 1)].sum(0) + Cb[m * (i - 1):m * i].sum(0)) / (2 * m)
        assert np.allclose(out[i], ref, atol=1e-12)
    # HCA with zero logits: mean of the block
    out = R.hca_fold(Ca, z, zb, m)
    assert np.allclose(out, Ca[: (n // m) * m].reshape(-1, m, c).mean(1), atol=1e-12)
    # a large positional bias on one in-block row picks that row (the bias enters the logits)
    for r in range(m):
        B = np.zeros((m, c))
        B[r] = 60.0
        out = R.hca_fold(Ca, z, B, m)
        assert np.allclose(out, Ca[r: (n // m) * m: m], atol=1e-12)
        out = R.csa_fold(Ca, Cb, z, z, B, zb, m)
        assert np.allclose(out, Ca[r: (n // m) * m: m], atol=1e-12)
        out = R.csa_fold(Ca, Cb, z, z, zb, B, m)
        assert np.allclose(out[1:], Cb[r: (n // m - 1) * m: m], atol=1e-12)
        assert np.allclose(out[0], Ca[0:m].mean(0), atol=1e-12)


def test_fold_dependency_matches_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_m4.json")))
    m = g["m"]
    dims = _dims(m=m)
    rng = np.random.default_rng(5)
    W = _weights(dims, rng)
    n = 4 * m
    H = rng.standard_normal((n, dims.d))
    base = R.compress_sequence(H, W, dims)["entry_pre"]
    reached = {j: set() for j in range(n)}
    for j in range(n):
        H2 = H.copy()
        H2[j] += rng.standard_normal(dims.d)
        out = R.compress_sequence(H2, W, dims)["entry_pre"]
        changed = np.where(np.abs(out - base).max(axis=1) > 1e-12)[0]
        reached[j] = set(changed.tolist())
    for e in g["entries"]:
        for j in e["a_tokens"] + e["b_tokens"]:
            assert e["i"] in reached[j]
    for j in range(n):
        expect = {i for i in (j // m, j // m + 1) if i < n // m}
        assert reached[j] == expect
        if j // m + 1 < n // m:
            assert len(reached[j]) == g["entries_per_token_csa"]


def test_hca_dependency_one_entry_per_token():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_m4.json")))["hca"]
    m = 8  # the structure does not depend on m'; a small block keeps the test quick
    dims = _dims(m=m, dual=False, top_k=0)
    rng = np.random.default_rng(6)
    W = _weights(dims, rng)
    n = 3 * m
    H = rng.standard_normal((n, dims.d))
    base = R.compress_sequence(H, W, dims)["entry_pre"]
    for j in range(n):
        H2 = H.copy()
        H2[j] += 1.0
        out = R.compress_sequence(H2, W, dims)["entry_pre"]
        changed = np.where(np.abs(out - base).max(axis=1) > 1e-12)[0]
        assert changed.tolist() == [j // m]
        assert len(changed) == g["entries_per_token_hca"]


def test_compress_entries_equals_whole_sequence():
    for dual in (True, False):
        dims = _dims(dual=dual, m=4 if dual else 8, top_k=4 if dual else 0)
        rng = np.random.default_rng(7)
        W = _weights(dims, rng)
        n = 6 * dims.m
        H = rng.standard_normal((n, dims.d))
        full = R.compress_sequence(H, W, dims)
        sel = [0, 1, 3, 5]
        part = R.compress_entries(lambda a, b: H[a:b], sel, W, dims)
        assert np.allclose(part["entry_fin"], full["entry_fin"][sel], atol=1e-12)
        if dual:
            assert np.allclose(part["ki_pre"], full["ki_pre"][sel], atol=1e-12)


def test_storage_layout_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "kv_storage.json")))
    dims = _dims(c=g["c"], rope_dim=g["rope_dim"], c_I=g["c_I"], m=g["m"], kv_fmt="q",
                 idx_fmt="e4m3", d=64)
    y = np.random.default_rng(8).standard_normal((3, g["c"]))
    vals, b = R.store_kv(y, dims)
    assert b.shape == (3, g["bytes_per_entry"])
    # elements kept per token by one CSA layer: (c + c_I) / m; by one HCA layer: c / m'
    n = 64 * g["m"]
    rng = np.random.default_rng(9)
    W = _weights(dims, rng)
    out = R.compress_sequence(rng.standard_normal((n, dims.d)), W, dims)
    per_tok = (out["entry"].size + out["ki"].size) / n
    assert per_tok == g["csa_elements_per_token"]
    assert g["c"] / g["m_prime"] == g["hca_elements_per_token"]
    # entries at a 1M context and positions covered by a Pro query
    assert abs(g["context_1m"] // g["m"] - g["csa_entries_at_1m_approx"]) / g["csa_entries_at_1m_approx"] < 0.01
    assert g["context_1m"] // g["m_prime"] == g["hca_entries_at_1m_approx"]
    assert g["pro_top_k"] * g["m"] == g["pro_tokens_covered_per_query_approx"]


# ----------------------------------------------------------------------------- norm / rope


def test_rmsnorm_unit_rms():
    x = np.random.default_rng(10).standard_normal((5, 64)) * 7
    y = R.rmsnorm(x, None, 1e-6)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-7)
    g = np.linspace(0.5, 2, 64)
    assert np.allclose(R.rmsnorm(x, g, 1e-6), g * y)


def test_rope_textbook_cases():
    r, c, base = 8, 12, 10000.0
    x = np.zeros(c)
    x[c - r] = 1.0  # first rotated pair, frequency base^0 = 1: turns by exactly pos radians
    for pos in (1, 5, -3):
        y = R.rope_rotate(x, pos, r, base)
        assert np.allclose(y[c - r:c - r + 2], [math.cos(pos), math.sin(pos)], atol=1e-15)
        assert np.all(y[: c - r] == 0)
    x = np.zeros(c)
    x[c - 2] = 1.0  # last pair, frequency base^(-(r-2)/r)
    y = R.rope_rotate(x, 7, r, base)
    th = 7 * base ** (-(r - 2) / r)
    assert np.allclose(y[c - 2:], [math.cos(th), math.sin(th)], atol=1e-15)
    # group laws R_p R_q = R_{p+q}, R_p^T = R_{-p}
    v = np.random.default_rng(11).standard_normal(c)
    assert np.allclose(R.rope_rotate(R.rope_rotate(v, 13, r, base), 29, r, base), R.rope_rotate(v, 42, r, base))
    assert np.allclose(R.rope_rotate(R.rope_rotate(v, 1000003, r, base), -1000003, r, base), v, atol=1e-9)


def test_single_key_output_is_relative_rotation():
    # One key at position p with no sink: weight 1, o = key, o~ = R_{-tau} R_p u = R_{p-tau} u.
    dims = _dims(c=16, rope_dim=8)
    rng = np.random.default_rng(12)
    u = rng.standard_normal(16)
    p, tau = 37, 101
    key = R.rope_rotate(u, p, dims.rope_dim, dims.rope_base)
    q = rng.standard_normal((dims.n_h, 16))
    out = R.attend(q, tau, key[None, :], None, None, dims)
    expect = R.rope_rotate(u, p - tau, dims.rope_dim, dims.rope_base)
    for h in range(dims.n_h):
        assert np.allclose(out[h], expect, atol=1e-12)


def test_shift_invariance_of_output():
    # Adding the same offset to every position (query, entries, window rows) leaves the
    # output unchanged: scores and outputs depend on relative positions only.
    dims = _dims(c=16, rope_dim=8)
    rng = np.random.default_rng(13)
    U = rng.standard_normal((9, 16))
    pos = np.array([0, 4, 8, 20, 21, 22, 23, 24, 25])
    q = rng.standard_normal((dims.n_h, 16))
    sink = rng.standard_normal(dims.n_h) * 0.3
    outs = []
    for shift in (0, 1000, 999983):
        keys = R.rope_rotate(U, pos + shift, dims.rope_dim, dims.rope_base)
        outs.append(R.attend(q, 25 + shift, keys, None, sink, dims))
    assert np.allclose(outs[0], outs[1], atol=1e-9)
    assert np.allclose(outs[0], outs[2], atol=1e-7)


# ----------------------------------------------------------------------------- indexer / top-k


def test_index_scores_closed_form_and_exactness():
    rng = np.random.default_rng(14)
    codes_q = codecs.e4m3_encode(rng.standard_normal((1, 64)) * 4)
    codes_k = codecs.e4m3_encode(rng.standard_normal((50, 64)) * 0.3)
    q, K = codecs.e4m3_decode(codes_q), codecs.e4m3_decode(codes_k)
    s = R.index_scores(q, np.ones(1), K)
    for j in range(50):
        exact = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q[0], K[j])), Fraction(0))
        assert s[j] == float(max(exact, Fraction(0)))  # bit-exact: dots of E4M3 values fit float64
    # MXFP4 operands (per-block scales differ): the dots are exact in float64 as well
    cq, sq = codecs.mxfp4_encode(rng.standard_normal((1, 128)) * 3)
    ck, sk = codecs.mxfp4_encode(rng.standard_normal((20, 128)) * np.array([0.05, 0.5, 2.0, 0.01]).repeat(32))
    q4 = codecs.mxfp4_decode(codecs.mxfp4_pack(cq), sq)
    K4 = codecs.mxfp4_decode(codecs.mxfp4_pack(ck), sk)
    s4 = R.index_scores(q4, np.ones(1), K4)
    for j in range(20):
        exact = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q4[0], K4[j])), Fraction(0))
        assert s4[j] == float(max(exact, Fraction(0)))
    # several heads: sum_h w_h ReLU(q_h . K_s)
    qh = rng.standard_normal((3, 64))
    w = np.array([0.5, -2.0, 1.25])
    s = R.index_scores(qh, w, K)
    for j in range(50):
        ref = sum(w[h] * max(0.0, float(np.dot(qh[h], K[j]))) for h in range(3))
        assert abs(s[j] - ref) <= 1e-12 * (1 + abs(ref))


def _bf16_nearest_exact(x: Fraction) -> float:
    """Nearest bfloat16 to the rational x (ties to the even bit pattern), by comparing exact
    distances to the bfloat16 values around x's float64 rounding."""
    c = np.float32(float(x))
    bits = int(np.array([c], np.float32).view(np.uint32)[0]) >> 16
    cands = []
    for b in (bits - 1, bits, bits + 1):
        if 0 <= b < 0x10000 and (b & 0x7F80) != 0x7F80:
            cands.append((b, float(np.array([b << 16], np.uint32).view(np.float32)[0])))
    best = min(cands, key=lambda bv: (abs(Fraction(bv[1]) - x), bv[0] & 1))
    return best[1]


def _mx(rng, shape, lo, hi):
    """Random MXFP4 rows: element codes, scale codes in lo .. hi, decoded exactly."""
    codes = rng.integers(0, 16, shape).astype(np.uint8)
    scales = rng.integers(lo, hi + 1, shape[:-1] + (shape[-1] // 32,)).astype(np.uint8)
    return codecs.mxfp4_decode(codecs.mxfp4_pack(codes), scales)


def test_bf16_index_scores_are_the_exact_score_rounded_once():
    """BF16 scores of the FP4 path: the exact score rounded once, even where the block scales
    span far more octaves than float64 holds (scale codes 80 .. 150: products of block scales
    from 2^-94 to 2^46)."""
    rng = np.random.default_rng(71)
    qI = _mx(rng, (4, 128), 80, 150)
    w = codecs.bf16_decode(codecs.bf16_encode(rng.standard_normal(4)))
    K = _mx(rng, (40, 128), 80, 150)
    K[3, 32:64] = 0.0                        # an all-zero block
    got = R.bf16_index_scores(qI, w, K)
    for j in range(K.shape[0]):
        exact = Fraction(0)
        for h in range(4):
            dot = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qI[h], K[j])), Fraction(0))
            exact += Fraction(float(w[h])) * max(dot, Fraction(0))
        assert got[j] == _bf16_nearest_exact(exact), j


def test_bf16_index_scores_decide_near_midpoints_exactly():
    """Crafted scores 1 + 2^-8 +- 2^-70: the first block gives the midpoint between the
    bfloat16 values 1 and 1 + 2^-7, a block 62 octaves further down decides the side.  float64
    drops the small term and rounds the tie to even (1.0) both times; the exact rounding goes
    up for + and down for -, and an exact tie goes to the even value."""
    def row(vals_by_block, scale_codes):
        codes = np.zeros(128, np.uint8)
        for blk, elems in vals_by_block.items():
            for i, code in elems:
                codes[32 * blk + i] = code
        return codecs.mxfp4_decode(codecs.mxfp4_pack(codes[None]), np.array([scale_codes], np.uint8))[0]
    # E2M1 code 2 is 1.0, code 10 is -1.0
    q = row({0: [(0, 2)], 1: [(0, 2)], 2: [(0, 2)]}, [127, 123, 87, 127])    # 1, 2^-4, 2^-40
    k_up = row({0: [(0, 2)], 1: [(0, 2)], 2: [(0, 2)]}, [127, 123, 97, 127])   # 1, 2^-4, 2^-30
    k_dn = row({0: [(0, 2)], 1: [(0, 2)], 2: [(0, 10)]}, [127, 123, 97, 127])
    k_tie = row({0: [(0, 2)], 1: [(0, 2)]}, [127, 123, 127, 127])
    K = np.stack([k_up, k_dn, k_tie])
    f64 = R.index_scores(q[None], np.ones(1), K)
    assert np.all(codecs.bf16_round_nearest(f64) == 1.0)          # what float64 would give
    got = R.bf16_index_scores(q[None], np.ones(1), K)
    assert got[0] == 1.0 + 2.0 ** -7 and got[1] == 1.0 and got[2] == 1.0


def _topk_bruteforce(scores, k):
    V = len(scores)
    if V <= k:
        return list(range(V))
    sel = []
    for s in range(V):
        better = sum(1 for t in range(V) if scores[t] > scores[s] or (scores[t] == scores[s] and t < s))
        if better < k:
            sel.append(s)
    return sel


def test_topk_bruteforce():
    rng = np.random.default_rng(15)
    for trial in range(60):
        V = int(rng.integers(1, 40))
        k = int(rng.integers(1, 12))
        if trial % 3 == 0:
            sc = rng.integers(-3, 4, V).astype(np.float64)  # many exact ties
        else:
            sc = rng.standard_normal(V)
        if trial % 5 == 0:
            sc[rng.integers(0, V)] = -0.0
            sc[rng.integers(0, V)] = 0.0
        got = R.topk(sc, k).tolist()
        assert got == _topk_bruteforce(sc, k)
        assert got == sorted(got)


def test_visibility_and_window():
    # the query's own block is never visible, even at its last token
    assert R.visible_entries(0, 4, 100) == 0
    assert R.visible_entries(3, 4, 100) == 0
    assert R.visible_entries(4, 4, 100) == 1
    assert R.visible_entries(7, 4, 100) == 1
    assert R.visible_entries(131072, 4, 32768) == 32768
    assert R.visible_entries(10 ** 6, 4, 5) == 5
    assert R.window_positions(3, 128).tolist() == [0, 1, 2, 3]
    w = R.window_positions(1000, 128)
    assert w[0] == 873 and w[-1] == 1000 and len(w) == 128


# ----------------------------------------------------------------------------- attention


def test_reduces_to_dense_causal_mqa():
    """m = 1, every entry selected, no sink, a one-token window, b path off: the keys of
    query tau are exactly rows 0..tau, so CSA is dense causal MQA with K = V."""
    for rope_dim in (0, 8):
        dims = _dims(m=1, top_k=10 ** 6, n_win=1, rope_dim=rope_dim, c=16, d=24, n_h=3)
        rng = np.random.default_rng(16 + rope_dim)
        W = _weights(dims, rng)
        W["B_b"] = np.full_like(W["B_b"], -np.inf)  # switch the b path off
        n = 11
        H = rng.standard_normal((n, dims.d))
        out = R.compress_sequence(H, W, dims)
        assert np.allclose(out["entry"][: n], out["raw"][: n], atol=1e-12)
        Q = rng.standard_normal((n, dims.n_h, dims.c))
        qI = rng.standard_normal((n, dims.n_hI, dims.c_I))
        wI = rng.standard_normal((n, dims.n_hI))
        mine = np.stack([
            R.query_step(t, Q[t], qI[t], wI[t], None, None, out["entry"], out["ki"],
                         lambda p: out["raw"][p], n, dims)[0] for t in range(n)])
        # library reference: torch SDPA, float64, causal, K = V broadcast over heads
        keys = torch.from_numpy(out["raw"])  # [n][c], already normalised and rotated
        qt = np.stack([R.rope_rotate(R.rmsnorm(Q[t], None, dims.eps), t, rope_dim, dims.rope_base)
                       for t in range(n)])  # [n][h][c]
        qt_t = torch.from_numpy(qt).permute(1, 0, 2)  # [h][n][c]
        kv = keys.unsqueeze(0).expand(dims.n_h, n, dims.c)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt_t, kv, kv, is_causal=True, scale=dims.softmax_scale).permute(1, 0, 2).numpy()
        ref = np.stack([R.rope_rotate(ref[t], -t, rope_dim, dims.rope_base) for t in range(n)])
        assert np.allclose(mine, ref, atol=1e-12, rtol=1e-10)


def test_sink_properties():
    dims = _dims(c=16, rope_dim=8)
    rng = np.random.default_rng(20)
    keys = rng.standard_normal((7, 16))
    qt = rng.standard_normal((dims.n_h, 16))
    sink = np.array([-1.0, 0.0, 2.0])
    s = R.attention_weights(qt, keys, sink, dims)
    tot = s.sum(axis=1)
    z = dims.softmax_scale * qt @ keys.T
    e = np.exp(z).sum(axis=1)
    assert np.all(tot < 1.0)
    assert np.allclose(tot, e / (e + np.exp(sink)), atol=1e-14)  # 1 - e^{z'}/D
    assert np.allclose(R.attention_weights(qt, keys, None, dims).sum(axis=1), 1.0, atol=1e-14)
    assert np.allclose(R.attention_weights(qt, keys, np.full(3, -1e4), dims),
                       R.attention_weights(qt, keys, None, dims), atol=1e-14)
    q = rng.standard_normal((dims.n_h, 16))
    big = R.attend(q, 5, keys, None, np.full(3, 80.0), dims)
    assert np.abs(big).max() < 1e-30


def test_dense_equals_sparse_when_k_covers_all():
    dims = _dims(top_k=64, n_win=4)
    rng = np.random.default_rng(21)
    W = _weights(dims, rng)
    n = 40
    H = rng.standard_normal((n, dims.d))
    out = R.compress_sequence(H, W, dims)
    dense = R.Dims(**{**dims.__dict__, "top_k": 0})
    q = rng.standard_normal((dims.n_h, dims.c))
    qI = rng.standard_normal((dims.n_hI, dims.c_I))
    wI = rng.standard_normal(dims.n_hI)
    sink = rng.standard_normal(dims.n_h)
    for tau in (0, 3, 4, 17, 39):
        a = R.query_step(tau, q, qI, wI, None, sink, out["entry"], out["ki"], lambda p: out["raw"][p], n // 4, dims)
        b = R.query_step(tau, q, qI, wI, None, sink, out["entry"], out["ki"], lambda p: out["raw"][p], n // 4, dense)
        assert np.array_equal(a[1], b[1])
        assert np.allclose(a[0], b[0], atol=1e-14)
