"""Pins of the oracle's CSA2 pieces (the V4.1-Flash layer of PaperTrace "02 · DeepSeek-V4:
压缩注意力撑起 1M 上下文" §6.4): the single-path fold without bias, index keys projected from
the main entry, the MXFP4 main-KV row codec, and the layer as a whole.

Each test checks the oracle against something other than itself: closed forms, invariants
the reading implies, hand-worked MXFP4 blocks, brute-force selection, and torch SDPA in float64
for the m = 1 reduction.
"""
import math

import numpy as np
import torch

from oracle import codecs
from oracle import csa_ref as R


def _dims(**kw):
    base = dict(d=32, c=64, rope_dim=16, n_h=3, c_I=8, n_hI=2, m=4, dual=False, top_k=4, n_win=4)
    base.update(kw)
    return R.Dims(**base)


def _weights(dims, rng):
    d, c, cI = dims.d, dims.c, dims.c_I
    return {"kv": rng.standard_normal((c, d)) / math.sqrt(d), "z": rng.standard_normal((c, d)) / math.sqrt(d),
            "B": None, "w_ik": rng.standard_normal((cI, c)) / math.sqrt(c), "gamma_kv": None}


def test_single_path_fold_closed_forms():
    """No bias and no overlap: zero logits give the plain mean of the entry's own m rows; a
    dominant logit picks its row; the weights of a column sum to 1."""
    rng = np.random.default_rng(40)
    n, c, m = 24, 6, 4
    C = rng.standard_normal((n, c))
    out = R.hca_fold(C, np.zeros((n, c)), None, m)
    assert np.allclose(out, C.reshape(-1, m, c).mean(1), atol=1e-14)
    for r in range(m):
        Z = np.zeros((n, c))
        Z[r::m] = 80.0
        assert np.allclose(R.hca_fold(C, Z, None, m), C[r::m], atol=1e-14)
    Z = rng.standard_normal((n, c)) * 4
    _, S = R.hca_fold(C, Z, None, m, return_weights=True)
    assert np.allclose(S.sum(axis=1), 1.0, atol=1e-14)
    # the softmax is over the rows of one column: a per-column shift of the logits changes nothing
    shift = rng.standard_normal(c) * 10
    assert np.allclose(R.hca_fold(C, Z + shift, None, m), R.hca_fold(C, Z, None, m), atol=1e-12)


def test_csa2_entry_depends_on_its_own_block_only():
    """Without the overlapping windows each token reaches exactly one entry (its own block),
    unlike CSA where a token also reaches the next entry through the b path."""
    dims = _dims()
    rng = np.random.default_rng(41)
    W = _weights(dims, rng)
    n = 5 * dims.m
    H = rng.standard_normal((n, dims.d))
    base = R.compress_sequence(H, W, dims)
    for j in range(n):
        H2 = H.copy()
        H2[j] += 1.0
        out = R.compress_sequence(H2, W, dims)
        for key in ("entry_pre", "ki_pre"):
            changed = np.where(np.abs(out[key] - base[key]).max(axis=1) > 1e-12)[0]
            assert changed.tolist() == [j // dims.m], (key, j)


def test_index_keys_from_entries():
    """K^I = RMSNorm(entry) W^IK: linear in the normalised entry (closed form with a selection
    matrix), blind to the entry's scale (the norm comes first), and carrying no position (no
    RoPE: the same folded entry gives the same key wherever it sits)."""
    dims = _dims()
    rng = np.random.default_rng(42)
    pre = rng.standard_normal((5, dims.c)) * 3
    # a selection matrix picks normalised dims 0, 2, ..., 14
    Wsel = np.zeros((dims.c_I, dims.c))
    Wsel[np.arange(dims.c_I), 2 * np.arange(dims.c_I)] = 1.0
    rms = np.sqrt(np.mean(pre * pre, axis=1, keepdims=True) + dims.eps)
    assert np.allclose(R.index_keys_from_entries(pre, Wsel, None, dims), (pre / rms)[:, ::2][:, :dims.c_I],
                       atol=1e-14)
    W = rng.standard_normal((dims.c_I, dims.c))
    k = R.index_keys_from_entries(pre, W, None, dims)
    assert np.allclose(R.index_keys_from_entries(7.5 * pre, W, None, dims), k, atol=1e-10)
    # gamma scales the normalised dims before the projection
    g = rng.uniform(0.5, 2.0, dims.c)
    assert np.allclose(R.index_keys_from_entries(pre, W, g, dims), R.index_keys_from_entries(pre, W * g, None, dims),
                       atol=1e-12)
    # position-free: the keys of a compressed sequence equal those of its entries moved to any position
    Wl = _weights(dims, rng)
    H = rng.standard_normal((3 * dims.m, dims.d))
    out = R.compress_sequence(H, Wl, dims)
    assert np.allclose(out["ki_pre"], R.index_keys_from_entries(out["entry_pre"], Wl["w_ik"], None, dims),
                       atol=1e-14)
    moved = R.compress_entries(lambda a, b: np.concatenate([np.zeros((8 * dims.m, dims.d)), H])[a:b],
                               [8, 9, 10], Wl, dims)
    assert np.allclose(moved["ki_pre"], out["ki_pre"], atol=1e-12)
    assert not np.allclose(moved["entry_fin"], out["entry_fin"], atol=1e-6)   # the entries do rotate


def test_mxfp4_main_rows_worked_blocks():
    """The FP4 main row: non-RoPE dims as MXFP4 blocks of 32 (OCP MX rule), RoPE dims bf16.
    Worked blocks: max 6 -> scale 2^0 and exact elements; max 5 -> scale 2^0, 5 rounds to 4
    (tie at 5 between 4 and 6 goes to the even significand 4); max 0.75 -> floor(log2 0.75) =
    -1, scale 2^-3, 0.75 = 6 x 2^-3 exact; an all-zero block -> scale code 127 and zeros."""
    dims = _dims(c=160, rope_dim=32, kv_fmt="q4")        # 128 non-RoPE dims = 4 blocks
    y = np.zeros((1, 160))
    y[0, 0:4] = [6.0, -3.0, 1.5, 0.5]
    y[0, 32:35] = [5.0, 1.0, -2.5]
    y[0, 64:66] = [0.75, 0.25]
    y[0, 128:] = np.linspace(-2, 2, 32)
    vals, b = R.store_kv(y, dims)
    assert b.shape == (1, 64 + 4 + 64)
    scales = b[0, 64:68]
    assert scales.tolist() == [127, 127, 124, 127]
    assert vals[0, 0:4].tolist() == [6.0, -3.0, 1.5, 0.5]
    assert vals[0, 32:35].tolist() == [4.0, 1.0, -2.0]   # 5 -> 4 (tie to even); -2.5 -> -2 (tie to even)
    assert vals[0, 64:66].tolist() == [0.75, 0.25]
    assert np.all(vals[0, 96:128] == 0.0)
    assert np.array_equal(vals[0, 128:], codecs.bf16_decode(codecs.bf16_encode(y[0, 128:])))
    # nibble order: element 2i in the low nibble of byte i
    assert b[0, 0] == (codecs.e2m1_encode_scaled(np.array([6.0]), np.array([0]))[0]
                       | (codecs.e2m1_encode_scaled(np.array([-3.0]), np.array([0]))[0] << 4))


def test_mxfp4_main_rows_error_bound():
    """The MX rule puts a block's maximum in [4, 8) x 2^e.  Below 6 x 2^e an element is off
    by at most half an E2M1 step (the largest step, between 4 and 6, is 2 x 2^e); above it
    the element saturates at 6 x 2^e: |v - y| <= max(2^e, |y| - 6 x 2^e) < 2 x 2^e."""
    dims = _dims(c=512, rope_dim=64, kv_fmt="q4")
    y = np.random.default_rng(43).standard_normal((50, 512)) * np.exp(np.random.default_rng(44).uniform(-4, 4, (50, 1)))
    vals, b = R.store_kv(y, dims)
    e = b[:, 224:238].astype(np.int64) - 127
    err = np.abs(vals[:, :448] - y[:, :448]).reshape(50, 14, 32)
    ay = np.abs(y[:, :448]).reshape(50, 14, 32)
    step = np.ldexp(1.0, e)[..., None]
    assert np.all(err <= np.maximum(step, ay - 6 * step))
    assert np.all(err < 2 * step)
    amax = ay.max(-1)
    assert np.all(amax < 8.0 * np.ldexp(1.0, e))
    assert np.all(amax >= 4.0 * np.ldexp(1.0, e))


def test_csa2_reduces_to_dense_causal_mqa():
    """m = 1, every entry selected, no sink, a one-token window: each entry is its token's
    finalized row (a softmax over one logit is 1), so CSA2 is dense causal MQA with K = V."""
    for rope_dim in (0, 8):
        dims = _dims(m=1, top_k=10 ** 6, n_win=1, rope_dim=rope_dim, c=16, d=24)
        rng = np.random.default_rng(45 + rope_dim)
        W = _weights(dims, rng)
        n = 9
        H = rng.standard_normal((n, dims.d))
        out = R.compress_sequence(H, W, dims)
        assert np.allclose(out["entry"], out["raw"], atol=1e-12)
        Q = rng.standard_normal((n, dims.n_h, dims.c))
        qI = rng.standard_normal((n, dims.n_hI, dims.c_I))
        wI = rng.standard_normal((n, dims.n_hI))
        mine = np.stack([R.query_step(t, Q[t], qI[t], wI[t], None, None, out["entry"], out["ki"],
                                      lambda p: out["raw"][p], n, dims)[0] for t in range(n)])
        qt = np.stack([R.rope_rotate(R.rmsnorm(Q[t], None, dims.eps), t, rope_dim, dims.rope_base) for t in range(n)])
        kv = torch.from_numpy(out["raw"]).unsqueeze(0).expand(dims.n_h, n, dims.c)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qt).permute(1, 0, 2), kv, kv, is_causal=True,
            scale=dims.softmax_scale).permute(1, 0, 2).numpy()
        ref = np.stack([R.rope_rotate(ref[t], -t, rope_dim, dims.rope_base) for t in range(n)])
        assert np.allclose(mine, ref, atol=1e-12, rtol=1e-10)


def test_csa2_selection_by_brute_force():
    """The CSA2 query step selects the top-k of the scores of the projected keys: checked by
    ranking every visible entry by hand on a small sequence."""
    dims = _dims(top_k=3, n_win=2)
    rng = np.random.default_rng(47)
    W = _weights(dims, rng)
    n = 9 * dims.m + 2
    out = R.compress_sequence(rng.standard_normal((n, dims.d)), W, dims)
    qI = rng.standard_normal((dims.n_hI, dims.c_I))
    wI = rng.standard_normal(dims.n_hI)
    q = rng.standard_normal((dims.n_h, dims.c))
    tau = n - 1
    _, sel, sc = R.query_step(tau, q, qI, wI, None, None, out["entry"], out["ki"], lambda p: out["raw"][p],
                              n // dims.m, dims)
    V = tau // dims.m
    manual = [sum(w * max(0.0, float(np.dot(qh, out["ki"][s]))) for qh, w in zip(qI, wI)) for s in range(V)]
    order = sorted(range(V), key=lambda s: (-manual[s], s))[:3]
    assert sorted(order) == sel.tolist()
    assert np.allclose(sc, manual, atol=1e-12)
