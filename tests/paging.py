"""Paged caches for the GPU tests: a shuffled block table over a page pool, and the moves
between a paged cache and the contiguous layout the checks read.

A page holds E = page_tokens / m entries; logical page j of sequence b is pool page
``block_table[b][j]``.  The table here is a random permutation of the pool's pages (a few
spare pages stay unused), so that neighbouring logical pages lie far apart in the pool.
"""
from types import SimpleNamespace

import numpy as np
import torch

import long_context_attention_11_amd as L


def paged_cache(dims, B: int, cap: int, win_cap: int, seed: int = 0, page_tokens: int = 128,
                spare: int = 5, device="cuda") -> "L.Cache":
    E = page_tokens // dims.m
    max_blocks = -(-cap // E)
    n_pages = B * max_blocks + spare
    perm = np.random.default_rng(seed).permutation(n_pages)[: B * max_blocks].astype(np.int32)
    bt = torch.from_numpy(perm.reshape(B, max_blocks)).to(device)
    return L.Cache(dims, B=B, cap=cap, win_cap=win_cap, device=device, block_table=bt,
                   page_tokens=page_tokens, n_pages=n_pages)


def _where(cache):
    """(pool page, row in page) of every logical entry, [B][cap] each."""
    E = cache.page_tokens // cache.dims.m
    i = torch.arange(cache.cap, device=cache.kv.device)
    bt = cache.block_table.long()
    return bt[:, i // E], (i % E).expand(cache.B, -1)


def _mx_split(ki, rows, cI):
    """An MXFP4 key tensor [groups][rows * (cI/2 + cI/32)] as (codes, scales) views."""
    n = rows * (cI // 2)
    return ki[:, :n].view(ki.shape[0], rows, cI // 2), ki[:, n:].view(ki.shape[0], rows, cI // 32)


def store_logical(cache, kv=None, ki=None):
    """Write contiguous-layout entries ([B][cap][row]) and keys (the contiguous cache's ki
    layout) into the cache, paged or not."""
    if cache.block_table is None:
        if kv is not None:
            cache.kv.copy_(kv)
        if ki is not None:
            cache.ki.copy_(ki.reshape(cache.ki.shape))
        return
    pg, rw = _where(cache)
    if kv is not None:
        cache.kv[pg, rw] = kv.to(cache.kv.device)
    if ki is not None:
        ki = ki.to(cache.ki.device)
        if cache.dims.idx_fmt == "mxfp4":
            cI = cache.dims.c_I
            lc, ls = _mx_split(ki.reshape(cache.B, -1), cache.cap, cI)
            pc, ps = _mx_split(cache.ki, cache.page_tokens // cache.dims.m, cI)
            pc[pg, rw] = lc
            ps[pg, rw] = ls
        else:
            cache.ki[pg, rw] = ki.reshape(cache.B, cache.cap, -1)


def logical(cache):
    """The cache in the contiguous layout (a copy for paged caches; the cache itself
    otherwise), with the attributes the checks read."""
    if cache.block_table is None:
        return cache
    pg, rw = _where(cache)
    kv = cache.kv[pg, rw]
    ki = codes = scales = None
    if cache.ki is not None:
        if cache.dims.idx_fmt == "mxfp4":
            pc, ps = _mx_split(cache.ki, cache.page_tokens // cache.dims.m, cache.dims.c_I)
            codes, scales = pc[pg, rw], ps[pg, rw]
            ki = torch.cat([codes.reshape(cache.B, -1), scales.reshape(cache.B, -1)], 1)
        else:
            ki = cache.ki[pg, rw]
    return SimpleNamespace(dims=cache.dims, B=cache.B, cap=cache.cap, win_cap=cache.win_cap, kv=kv, ki=ki,
                           ki_codes=codes, ki_scales=scales, n_entries=cache.n_entries, win=cache.win,
                           win_pos=cache.win_pos, state=cache.state, block_table=None)
