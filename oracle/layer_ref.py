"""CPU oracle of the projections around the attention core: the low-rank query path before it
and the grouped output projection after it.

TEST INFRASTRUCTURE ONLY, under the same rule as ``csa_ref``: imported by ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` only.  Plain float64
numpy written from the pages.

Sources:
  [RN] "DeepSeekV4技术报告阅读笔记" (zouxinn.github.io): §2.3.2 eqs. 13-15 (the shared
       query latent c^Q, the indexer queries and head weights), §2.3.3 eq. 18 (attention
       queries from the same latent) and its "Grouped Output Projection" paragraph; §2.4
       (HCA uses the same two projections).
  [DD] "DeepSeek-V4 架构设计深度解析" (blog.sysu-sam.com), stage three: g = 16 (Pro) / 8
       (Flash) groups, each projected to d_g = 1024.
  [PT] "02 · DeepSeek-V4: 压缩注意力撑起 1M 上下文" (PaperTrace, yayajjiang.github.io), §1:
       the query up-projection of Pro is 1536 x 128 x 512 (so d_c = 1536), about 1.0e8
       parameters; §2.2: g = 16 (Pro) / 8 (Flash), d_g = 1024, the grouped output projection
       about 1.8e8 parameters against about 4.7e8 ungrouped.

Weights follow the convention of ``csa_ref.project``: a matrix W in R^{a x b} is stored
transposed, [b][a], one row per output column.
  dq   [d_c][d]            W^DQ   (eq. 13)
  uq   [n_h * c][d_c]      W^UQ   (eq. 18)
  iuq  [n_hI * c_I][d_c]   W^IUQ  (eq. 14)
  w    [n_hI][d]           W^w    (eq. 15)
  og   [g][d_g][c n_h / g] the g group projections
  o    [d][g * d_g]        the projection of the concatenated groups to d

Readings (the pages name the maps, not their storage):
  * c^Q, like every activation that feeds a matrix product here, is held in bfloat16
    (rounded to nearest even from its float32 value); q and w are stored in bfloat16 and
    q^I in the indexer's format (E4M3, or MXFP4 in 32-blocks), as the path consumes them.
  * The concatenated group outputs [o'_1; ...; o'_g] are held in bfloat16 before the last
    projection; the layer output is bfloat16.
  * No normalisation or bias is applied to c^Q or to the group outputs (the pages write
    plain products).

Pins (tests/test_oracle_layer_pins.py): the grouped projection equals one product with the
block-diagonal matrix of the group maps followed by the last map; g = 1 with an identity
group map is the ungrouped projection; the attention and indexer queries come from the same
latent (eq. 14 and eq. 18 with equal up-projections agree); an identity down-projection
passes h through; scaling h scales every output; the weight shapes reproduce the parameter
counts the pages print for Pro (tests/golden/projection_sizes.json).
"""
from __future__ import annotations

import numpy as np

from . import codecs
from .csa_ref import Dims, store_index_keys

__all__ = ["projection_shapes", "to_bf16", "query_projections", "grouped_output_projection"]


def projection_shapes(dims: Dims, d_c: int, g: int, d_g: int) -> dict:
    """Stored shapes of the six weight matrices (transposed convention above)."""
    if (dims.n_h * dims.c) % g:
        raise ValueError("n_h * c must split into g equal groups")
    return {
        "dq": (d_c, dims.d),
        "uq": (dims.n_h * dims.c, d_c),
        "iuq": (dims.n_hI * dims.c_I, d_c),
        "w": (dims.n_hI, dims.d),
        "og": (g, d_g, dims.n_h * dims.c // g),
        "o": (dims.d, g * d_g),
    }


def to_bf16(x) -> np.ndarray:
    """The bfloat16 value of x (nearest even from its float32 value), as float64."""
    return codecs.bf16_decode(codecs.bf16_encode(x))


def query_projections(h, W: dict, dims: Dims) -> dict:
    """[RN] eqs. 13-15 and 18 for the rows of h ([T][d]).

    c^Q = h W^DQ (eq. 13) is the latent shared by both query sets; q^I = c^Q W^IUQ
    (eq. 14), w^I = h W^w (eq. 15), q = c^Q W^UQ (eq. 18).  Returns float64 values before
    storage ("q_pre", "qI_pre", "w_pre", and the bfloat16 latent "cQ") and the stored ones:
    "q" and "w" (bfloat16 values), "qI" (values in the indexer's format) with "qI_bytes"."""
    h = np.asarray(h, np.float64)
    cQ = to_bf16(h @ np.asarray(W["dq"], np.float64).T)
    q_pre = cQ @ np.asarray(W["uq"], np.float64).T
    qI_pre = cQ @ np.asarray(W["iuq"], np.float64).T
    w_pre = h @ np.asarray(W["w"], np.float64).T
    T = h.shape[0]
    qI_rows = qI_pre.reshape(T, dims.n_hI, dims.c_I)
    qI, qI_bytes = store_index_keys(qI_rows, dims)
    return {
        "cQ": cQ,
        "q_pre": q_pre.reshape(T, dims.n_h, dims.c),
        "qI_pre": qI_rows,
        "w_pre": w_pre,
        "q": to_bf16(q_pre).reshape(T, dims.n_h, dims.c),
        "qI": qI,
        "qI_bytes": qI_bytes,
        "w": to_bf16(w_pre),
    }


def grouped_output_projection(o, W: dict, g: int) -> dict:
    """The grouped output projection ([RN] §2.3.3; [DD] stage three) of the attention output
    o ([T][n_h c], heads in order): the heads form g consecutive groups of n_h / g heads;
    group i's c n_h / g values are projected to d_g by its own map, the g results are
    concatenated and projected to d.  Returns the concatenated group outputs before and
    after bfloat16 storage ("mid_pre", "mid") and the output before and after ("out_pre",
    "out")."""
    o = np.asarray(o, np.float64)
    og = np.asarray(W["og"], np.float64)
    T, width = o.shape
    G = width // g
    parts = []
    for i in range(g):
        parts.append(o[:, i * G:(i + 1) * G] @ og[i].T)
    mid_pre = np.concatenate(parts, axis=1)
    mid = to_bf16(mid_pre)
    out_pre = mid @ np.asarray(W["o"], np.float64).T
    return {"mid_pre": mid_pre, "mid": mid, "out_pre": out_pre, "out": to_bf16(out_pre)}
