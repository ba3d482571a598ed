"""Pins of the oracle's query and grouped output projections (oracle/layer_ref.py) against
what the pages and the algebra fix, independent of the oracle's own loops."""
import json
import os

import numpy as np
import scipy.linalg

from oracle import layer_ref as LR
from oracle.csa_ref import Dims

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dims(**over):
    base = dict(d=12, c=8, rope_dim=4, n_h=4, c_I=8, n_hI=4, m=4, dual=True, top_k=4, n_win=4,
                kv_fmt="q", idx_fmt="e4m3")
    base.update(over)
    return Dims(**base)


def _ints(rng, shape, lo=-3, hi=3):
    # small integers: every product and sum below stays an integer under 256, so exact in
    # bfloat16 and no storage rounding blurs the comparisons
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


def test_grouped_projection_is_block_diagonal_product():
    """Grouping = one product with the block-diagonal matrix of the g group maps (heads in
    order, [RN] §2.3.3), then the map to d."""
    rng = np.random.default_rng(3)
    T, n_h, c, g, d_g, d = 3, 4, 2, 2, 3, 5
    G = n_h * c // g
    o = _ints(rng, (T, n_h * c), -2, 2)
    W = {"og": _ints(rng, (g, d_g, G), -1, 1), "o": _ints(rng, (d, g * d_g), -1, 1)}
    r = LR.grouped_output_projection(o, W, g)
    blk = scipy.linalg.block_diag(*[W["og"][i].T for i in range(g)])   # [n_h c][g d_g]
    assert blk.shape == (n_h * c, g * d_g)
    np.testing.assert_array_equal(r["mid_pre"], o @ blk)
    np.testing.assert_array_equal(r["out_pre"], (o @ blk) @ W["o"].T)
    # swapping two groups' maps changes the result (the group order matters)
    W2 = {"og": W["og"][::-1].copy(), "o": W["o"]}
    assert not np.array_equal(LR.grouped_output_projection(o, W2, g)["mid_pre"], r["mid_pre"])


def test_one_group_with_identity_map_is_the_ungrouped_projection():
    """g = 1 and d_g = c n_h with the identity group map: the direct projection o W^O."""
    rng = np.random.default_rng(4)
    T, width, d = 4, 6, 5
    o = _ints(rng, (T, width))
    Wo = _ints(rng, (d, width), -2, 2)
    r = LR.grouped_output_projection(o, {"og": np.eye(width)[None], "o": Wo}, 1)
    np.testing.assert_array_equal(r["mid"], o)
    np.testing.assert_array_equal(r["out_pre"], o @ Wo.T)


def test_queries_share_the_latent():
    """Eqs. 14 and 18 up-project the same c^Q: equal up-projections give equal queries, and
    an identity down-projection (d_c = d) passes h through (bf16-exact h)."""
    rng = np.random.default_rng(5)
    dims = _dims(n_h=2, c=8, n_hI=2, c_I=8)
    d = dims.d
    h = _ints(rng, (3, d))
    up = _ints(rng, (16, d), -1, 1)
    W = {"dq": np.eye(d), "uq": up, "iuq": up, "w": _ints(rng, (2, d), -1, 1)}
    r = LR.query_projections(h, W, dims)
    np.testing.assert_array_equal(r["cQ"], h)
    np.testing.assert_array_equal(r["q_pre"].reshape(3, -1), r["qI_pre"].reshape(3, -1))
    np.testing.assert_array_equal(r["q_pre"].reshape(3, -1), h @ up.T)
    np.testing.assert_array_equal(r["w_pre"], h @ W["w"].T)   # eq. 15 reads h, not c^Q


def test_query_outputs_scale_with_h():
    """Every map is linear and bfloat16 rounding commutes with scaling by 2: doubling h
    doubles c^Q, q, q^I (before storage) and w exactly."""
    rng = np.random.default_rng(6)
    dims = _dims()
    shapes = LR.projection_shapes(dims, d_c=6, g=2, d_g=3)
    W = {k: rng.standard_normal(shapes[k]) for k in ("dq", "uq", "iuq", "w")}
    h = rng.standard_normal((5, dims.d))
    a, b = LR.query_projections(h, W, dims), LR.query_projections(2 * h, W, dims)
    for key in ("cQ", "q_pre", "qI_pre", "w_pre", "q", "w"):
        np.testing.assert_array_equal(b[key], 2 * a[key])


def test_query_indexer_storage_formats():
    """q^I leaves in the indexer's storage: E4M3 codes, or MXFP4 (32-blocks) whose decoded
    values are within half a code of the latent's up-projection."""
    rng = np.random.default_rng(7)
    for fmt in ("e4m3", "mxfp4"):
        dims = _dims(c_I=32, n_hI=2, idx_fmt=fmt)
        shapes = LR.projection_shapes(dims, d_c=6, g=2, d_g=3)
        W = {k: rng.standard_normal(shapes[k]) for k in ("dq", "uq", "iuq", "w")}
        r = LR.query_projections(rng.standard_normal((4, dims.d)), W, dims)
        assert r["qI"].shape == (4, 2, 32)
        err = np.abs(r["qI"] - r["qI_pre"])
        # E4M3 keeps 3 mantissa bits, MXFP4 at least one below its block maximum
        rel = 2.0 ** -4 if fmt == "e4m3" else 0.25
        bound = rel * (np.abs(r["qI_pre"]) if fmt == "e4m3" else
                       np.abs(r["qI_pre"]).max(axis=-1, keepdims=True))
        assert np.all(err <= bound + 1e-300), fmt


def test_projection_sizes_match_the_pages():
    """The weight shapes reproduce the parameter counts printed for Pro."""
    gold = json.load(open(os.path.join(GOLDEN, "projection_sizes.json")))
    p = gold["pro"]
    dims = _dims(d=p["d"], n_h=p["n_h"], c=p["c"], n_hI=p["n_hI"], c_I=p["c_I"])
    shapes = LR.projection_shapes(dims, p["d_c"], p["g"], p["d_g"])
    n = {k: int(np.prod(v)) for k, v in shapes.items()}

    def two_digits(x):
        return float(f"{x:.2g}")

    assert two_digits(n["uq"]) == gold["query_up_params_approx"]
    assert two_digits(n["og"] + n["o"]) == gold["grouped_output_params_approx"]
    assert two_digits(p["n_h"] * p["c"] * p["d"]) == gold["ungrouped_output_params_approx"]
    # each group covers c n_h / g = 4096 of the 65536 head dims
    assert shapes["og"] == (16, 1024, 4096)
