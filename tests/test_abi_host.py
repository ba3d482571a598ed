"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports every symbol
include/csa.h declares, and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

import long_context_attention_11_amd as L
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "csa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    if not os.path.exists(L.lib_path()):
        pytest.skip("libcsa.so not built")
    lib = L.load()
    declared = _declared_symbols()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), f"libcsa.so does not export {name}"
    assert set(L.EXPORTED_SYMBOLS) == set(declared)
    assert L.csa_abi_version() == L.ABI_VERSION == 2


def _lib():
    if not os.path.exists(L.lib_path()):
        pytest.skip("libcsa.so not built")
    return L.load()


def test_sizes_follow_the_storage_layout():
    _lib()
    d2 = L.Dims.from_config(synth.config("c2"))
    assert L.csa_row_bytes(d2) == 576  # 448 E4M3 + 64 bf16
    assert L.csa_state_rows(d2) == 8 and L.csa_state_width(d2) == 4 * 512 + 4 * 128
    d1 = L.Dims.from_config(synth.config("c1"))
    assert L.csa_row_bytes(d1) == 4 * 64
    d5 = L.Dims.from_config(synth.config("c5"))
    assert L.csa_state_rows(d5) == 128 and L.csa_state_width(d5) == 2 * 512


def _status(fn, *args):
    return fn(*args)


def test_invalid_dims_are_rejected_on_the_host():
    lib = _lib()
    bad = [
        dict(c=63),                      # odd c
        dict(rope_dim=70),               # rope_dim > c
        dict(top_k=0),                   # CSA needs top_k
        dict(n_win=2),                   # n_win < m
        dict(top_k=-1),                  # negative top_k
        dict(dual=False, c_I=0),         # CSA2 (single path with top_k > 0) without index keys
    ]
    for over in bad:
        d = L.Dims.from_config(synth.config("c1"), **over)
        out = ctypes.c_size_t(0)
        st = lib.csa_workspace_size(ctypes.byref(d.struct()), L.OP_COMPRESS, 1, 1, 1, 1, 0,
                                    ctypes.byref(out))
        assert st == 1, over
        assert lib.csa_last_error().decode()
    # CSA2 (single path with an indexer) is a valid layer at both shapes, with FP4 main rows
    for name in ("c1v2", "c6", "c6fp4"):
        d = L.Dims.from_config(synth.config(name))
        out = ctypes.c_size_t(0)
        assert lib.csa_workspace_size(ctypes.byref(d.struct()), L.OP_FORWARD, 2, 1, 1, 64, 0,
                                      ctypes.byref(out)) == 0, lib.csa_last_error()
    assert L.csa_row_bytes(L.Dims.from_config(synth.config("c6"))) == 384 == synth.row_bytes(synth.config("c6"))
    # HCA too: a window shorter than m' would leave the open block's older tokens unseen
    d = L.Dims.from_config(synth.config("c5"), n_win=64)
    out = ctypes.c_size_t(0)
    assert lib.csa_workspace_size(ctypes.byref(d.struct()), L.OP_ATTEND, 1, 1, 1, 1, 0,
                                  ctypes.byref(out)) == 1
    assert "n_win" in lib.csa_last_error().decode()
    # an unbuilt combination: quantized rows need c = 512
    d = L.Dims.from_config(synth.config("c2"), c=256)
    out = ctypes.c_size_t(0)
    assert lib.csa_workspace_size(ctypes.byref(d.struct()), L.OP_COMPRESS, 1, 1, 1, 1, 0,
                                  ctypes.byref(out)) == 2


def test_null_and_workspace_errors_without_a_device():
    """Argument errors return before any HIP call, so they can be forced on a CPU host."""
    lib = _lib()
    d = L.Dims.from_config(synth.config("c2"))
    ds = d.struct()
    # NULL cache
    st = lib.csa_compress(ctypes.byref(ds), None, None, None, 1, None, None, 0, None)
    assert st == 1
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: checks fail before any launch
    cache = L._Cache(2, 64, 128, fake, fake, fake, fake, fake, fake)
    w = L._Weights(fake, fake, fake, fake, None)
    # T = 0
    assert lib.csa_compress(ctypes.byref(ds), ctypes.byref(w), ctypes.byref(cache), fake, 0, fake,
                            fake, 1 << 30, None) == 1
    # workspace too small
    assert lib.csa_compress(ctypes.byref(ds), ctypes.byref(w), ctypes.byref(cache), fake, 4, fake,
                            fake, 16, None) == 3
    # win_cap < n_win
    small = L._Cache(2, 64, 64, fake, fake, fake, fake, fake, fake)
    assert lib.csa_attend(ctypes.byref(ds), ctypes.byref(small), fake, None, None, fake, fake, 1,
                          fake, fake, fake, 1 << 30, None) == 1
    # HCA has no indexer
    d5 = L.Dims.from_config(synth.config("c5")).struct()
    assert lib.csa_index_topk(ctypes.byref(d5), ctypes.byref(cache), fake, fake, fake, fake, 1, fake,
                              None, fake, 1 << 30, None) == 1
    # a top_k larger than one selection workgroup's share is not built
    dk = L.Dims.from_config(synth.config("c2"), top_k=20000).struct()
    assert lib.csa_index_topk(ctypes.byref(dk), ctypes.byref(cache), fake, fake, fake, fake, 1, fake,
                              None, fake, 1 << 40, None) == 2
    # forward needs a ring that holds the chunk's window
    assert lib.csa_forward(ctypes.byref(ds), ctypes.byref(w), ctypes.byref(cache), fake, 64, fake,
                           fake, fake, fake, None, None, fake, None, fake, 1 << 30, None) == 1
    assert lib.csa_status_string(3) == b"workspace too small"
    # CSA2 needs its entry-to-key projection in w_idx (and takes no bias)
    d6 = L.Dims.from_config(synth.config("c6")).struct()
    no_ik = L._Weights(fake, None, None, None, None)
    assert lib.csa_compress(ctypes.byref(d6), ctypes.byref(no_ik), ctypes.byref(cache), fake, 4, fake,
                            fake, 1 << 30, None) == 1
    assert b"w_idx" in lib.csa_last_error()
    # the allocation-free forward: a 32768-token chunk needs more than its static scratch, which
    # it reports before any HIP call
    big = L._Cache(1, 270336, 32768 + 128, fake, fake, fake, fake, fake, fake)
    st = lib.csa_forward_noalloc(ctypes.byref(ds), ctypes.byref(w), ctypes.byref(big), fake, 32768, fake,
                                 fake, fake, fake, None, None, fake, fake, None)
    assert st == 3 and b"static" in lib.csa_last_error()
    assert L.csa_noalloc_scratch_bytes() == 64 << 20


def test_paged_cache_arguments_are_checked_on_the_host():
    """A block table brings page_tokens, max_blocks and n_pages, checked before any launch."""
    lib = _lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: checks fail before any launch
    w = L._Weights(fake, fake, fake, fake, None)

    def attend(cfg, cache):
        ds = L.Dims.from_config(cfg).struct()
        return lib.csa_attend(ctypes.byref(ds), ctypes.byref(cache), fake, None, None, fake, fake, 1,
                              None, fake, fake, 1 << 30, None)

    def paged(cap, max_blocks, page_tokens, n_pages):
        return L._Cache(2, cap, 128, fake, fake, fake, fake, fake, fake, fake, max_blocks, page_tokens, n_pages)

    c2, c5 = synth.config("c2"), synth.config("c5")
    # HCA: a page must hold whole entries of m' = 128 tokens, the table must reach cap
    for cache, msg in ((paged(64, 64, 100, 128), b"multiple of m"),
                       (paged(65, 64, 128, 128), b"cap exceeds"),
                       (paged(64, 0, 128, 128), b"max_blocks"),
                       (paged(64, 64, 128, 0), b"n_pages")):
        assert attend(c5, cache) == 1
        assert msg in lib.csa_last_error()
    # CSA with quantized keys: a page must hold a multiple of 16 entries
    ds = L.Dims.from_config(c2).struct()
    bad = paged(64, 32, 8, 64)                                # 2 entries per page
    assert lib.csa_index_topk(ctypes.byref(ds), ctypes.byref(bad), fake, fake, fake, fake, 1, fake,
                              None, fake, 1 << 30, None) == 2
    assert b"% 16" in lib.csa_last_error()
    # float32 keys take any page size that is a multiple of m: the cache passes its checks and
    # the call fails on T = 0, which is checked after them
    d1 = L.Dims.from_config(synth.config("c1")).struct()
    assert lib.csa_compress(ctypes.byref(d1), ctypes.byref(w), ctypes.byref(paged(64, 64, 4, 128)), fake, 0,
                            fake, fake, 1 << 30, None) == 1
    assert b"T must" in lib.csa_last_error()


def test_workspace_sizes_are_consistent():
    _lib()
    d = L.Dims.from_config(synth.config("c2"))
    full = L.csa_workspace_size(d, L.OP_FORWARD, B=1, T=32768, cap=270336)
    chunked = L.csa_workspace_size(d, L.OP_FORWARD, B=1, T=32768, cap=270336, q_chunk=2048)
    assert chunked < full
    assert L.csa_workspace_size(d, L.OP_INDEX_TOPK, Q=16, cap=32768) >= 16 * 32768 * 4


def test_projection_entry_points_reject_bad_arguments():
    """csa_query_project / csa_output_project: argument checks fail on the host."""
    lib = _lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: checks fail before any launch
    d2 = L.Dims.from_config(synth.config("c2")).struct()

    def pw(d_c=1536, g=8, d_g=1024):
        return L._ProjWeights(fake, fake, fake, fake, fake, fake, d_c, g, d_g)

    ok = pw()
    need = lib.csa_query_project_workspace_size(ctypes.byref(d2), ctypes.byref(ok), 16)
    assert need > 0
    # widths the GEMM tiles do not take, and a g that does not divide the heads
    for bad in (pw(d_c=100), pw(g=3), pw(d_g=1000), pw(g=0)):
        assert lib.csa_query_project(ctypes.byref(d2), ctypes.byref(bad), fake, 16, fake, fake, fake, fake,
                                     1 << 40, None) == 2
        assert lib.csa_query_project_workspace_size(ctypes.byref(d2), ctypes.byref(bad), 16) == 0
    # T = 0, missing outputs, too little workspace
    assert lib.csa_query_project(ctypes.byref(d2), ctypes.byref(ok), fake, 0, fake, fake, fake, fake,
                                 1 << 40, None) == 1
    assert lib.csa_query_project(ctypes.byref(d2), ctypes.byref(ok), fake, 16, fake, None, fake, fake,
                                 1 << 40, None) == 1
    assert lib.csa_query_project(ctypes.byref(d2), ctypes.byref(ok), fake, 16, fake, fake, fake, fake,
                                 need - 1, None) == 3
    # fp32 activations are not built for the projections
    d1 = L.Dims.from_config(synth.config("c1")).struct()
    assert lib.csa_output_project(ctypes.byref(d1), ctypes.byref(pw(d_c=64, g=4, d_g=64)), fake, 4, fake,
                                  fake, 1 << 40, None) == 2
    need_o = lib.csa_output_project_workspace_size(ctypes.byref(d2), ctypes.byref(ok), 16)
    assert need_o > 0
    assert lib.csa_output_project(ctypes.byref(d2), ctypes.byref(ok), fake, 16, None, fake, 1 << 40, None) == 1
    assert lib.csa_output_project(ctypes.byref(d2), ctypes.byref(ok), fake, 16, fake, fake, need_o - 1,
                                  None) == 3
