"""Host-side checks of libkvq.so: it loads, exports every symbol include/kvq.h
declares, carries the same codebook the oracle derives independently, sizes the
layout as specified, and rejects invalid calls on the host before any GPU work
(these calls never reach HIP, so they run without a GPU)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from packed_cache_attention_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_match_header():
    hdr = open(os.path.join(ROOT, "include", "kvq.h")).read()
    declared = set(re.findall(r"^\s*(?:int32_t|int64_t|const char \*)\s*(kvq_\w+)\(", hdr, re.M))
    assert declared == set(kvq.EXPORTS)
    L = kvq.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert L.kvq_version() == 1


@pytest.mark.parametrize("w", range(1, 9))
def test_codebook_matches_oracle(w):
    lev, thr, dd = kvq.get_codebook(w)
    cb = oracle.codebook(w)
    np.testing.assert_array_equal(lev, cb["levels_fp16"])
    np.testing.assert_array_equal(thr, cb["thresholds"])
    np.testing.assert_array_equal(dd, oracle.tables()["dD"])
    # the quantizers take a code's top bit as the sign test x >= 0: the middle threshold
    # of every width is exactly +0 (the levels are symmetric)
    mid = thr[1 << (w - 1)]
    assert mid == 0.0 and not np.signbit(mid)


@pytest.mark.parametrize("kb,vb", [(192, 3), (128, 2), (192, 2), (1024, 16), (0, 1), (300, 8), (7, 5)])
def test_layout_sizes(kb, vb):
    g = kvq.geom(3, kb, vb, 640)
    assert kvq.tile_bytes(g) == oracle.tile_bytes(128, kb, vb)
    assert kvq.cache_bytes(g) == 3 * 10 * oracle.tile_bytes(128, kb, vb)


def test_workspace_bytes_and_plan():
    g = kvq.geom(2, 192, 3, 131072)
    ws = kvq.decode_workspace_bytes(g, 16, 1, 131072)
    assert ws > 0 and ws % 4 == 0
    ws2 = kvq.decode_workspace_bytes(g, 16, 1, 131072, kvq.DECODE_GENERIC, 8)
    # the generic kernel's partials, then its query table (per sequence and KV head, 128
    # fields x the group padded to 4, 8 or 16 heads)
    assert ws2 == 1 * 16 * (2048 // 8) * 130 * 4 + 1 * 2 * 128 * 8 * 4
    ws3 = kvq.decode_workspace_bytes(g, 16, 1, 131072, kvq.DECODE_MFMA, 8)
    assert ws3 == 1 * 16 * (2048 // 8) * 130 * 4
    # the window call's workspace grows by whole chunks, the table once
    w = kvq.window_workspace_bytes(g, 128, 16, 1, 131072 + 128, kvq.DECODE_GENERIC, 8)
    assert w == 1 * 16 * (2048 // 8 + 4) * 130 * 4 + 1 * 2 * 128 * 8 * 4
    assert kvq.decode_workspace_bytes(g, 16, 1, 0) >= 0


def _st(r):
    return int(r)


FAKE = 1 << 20  # a non-null, 16-byte aligned address that is never dereferenced


def test_host_validation_rejects_before_gpu():
    L = kvq.lib()
    good = kvq.geom(2, 192, 3, 1024)
    st = L.kvq_block_energy(None, FAKE, 10, 256, 128, FAKE, None)
    assert st == -1
    bad = kvq.geom(2, 192, 3, 1024)
    bad.layout_version = 2
    assert L.kvq_block_energy(C.byref(bad), FAKE, 10, 256, 128, FAKE, None) == -8
    bad = kvq.geom(2, 192, 3, 1024, head_dim=7)
    assert L.kvq_block_energy(C.byref(bad), FAKE, 10, 256, 128, FAKE, None) == -2
    bad = kvq.geom(2, 600, 3, 1024)
    assert L.kvq_block_energy(C.byref(bad), FAKE, 10, 256, 128, FAKE, None) == -3
    bad = kvq.geom(2, 192, 9, 1024)
    assert L.kvq_block_energy(C.byref(bad), FAKE, 10, 256, 128, FAKE, None) == -3
    bad = kvq.geom(2, 192, 3, 1000)
    assert L.kvq_block_energy(C.byref(bad), FAKE, 10, 256, 128, FAKE, None) == -5
    # misaligned input / odd stride / null energy / negative count
    assert L.kvq_block_energy(C.byref(good), FAKE + 2, 10, 256, 128, FAKE, None) == -4
    assert L.kvq_block_energy(C.byref(good), FAKE, 10, 255, 128, FAKE, None) == -4
    assert L.kvq_block_energy(C.byref(good), FAKE, 10, 256, 128, None, None) == -1
    assert L.kvq_block_energy(C.byref(good), FAKE, -1, 256, 128, FAKE, None) == -1
    assert L.kvq_block_energy(C.byref(good), FAKE, 0, 256, 128, FAKE, None) == 0  # nothing to do
    # allocation: budgets and modes
    for budget, mode, want in ((513, 0, -3), (-1, 0, -3), (100, 1, -3), (192, 2, -1), (1024, 1, 0)):
        r = L.kvq_allocate_bits(C.byref(good), FAKE, 0 if want == 0 else 4, budget, mode, FAKE, FAKE, None)
        assert r == want, (budget, mode, r)
    # quantize: head_dim must be 128; capacity
    g64 = kvq.geom(2, 64, 3, 1024, head_dim=64)
    args = (FAKE, FAKE, 256, 128, 1, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert L.kvq_quantize_pack(C.byref(g64), *args) == -2
    args_cap = (FAKE, FAKE, 256, 128, 1, FAKE, FAKE, FAKE, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert L.kvq_quantize_pack(C.byref(good), *args_cap) == -5
    args_al = (FAKE + 2, FAKE, 255, 128, 1, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert L.kvq_quantize_pack(C.byref(good), *args_al) == -4
    # decode: GQA ratio, capacity, workspace, alignment
    d_args = lambda nq, max_len, ws, q=FAKE: (C.byref(good), nq, q, FAKE, FAKE, FAKE, 1, max_len, FAKE, FAKE, FAKE,
                                              0.1, FAKE, FAKE, ws, 0, 0, None)
    assert L.kvq_packed_decode_attn_ex(*d_args(3, 512, 1 << 30)) == -2
    assert L.kvq_packed_decode_attn_ex(*d_args(64, 512, 1 << 30)) == -2  # ratio 32 > 16
    assert L.kvq_packed_decode_attn_ex(*d_args(16, 2048, 1 << 30)) == -5
    assert L.kvq_packed_decode_attn_ex(*d_args(16, 512, 16)) == -6
    assert L.kvq_packed_decode_attn_ex(*d_args(16, 512, 1 << 30, q=FAKE + 8)) == -4
    assert kvq.status_string(-6) == "workspace too small"
    # decode step: the decode checks, then the new-token rows
    s_args = lambda kn, ss, ws=1 << 30: (C.byref(good), 16, FAKE, kn, FAKE, ss, 128, FAKE, FAKE, FAKE, 1, 512, FAKE,
                                         FAKE, FAKE, 0.1, FAKE, FAKE, ws, 0, 0, None)
    assert L.kvq_decode_step(*s_args(None, 256)) == -1
    assert L.kvq_decode_step(*s_args(FAKE + 2, 256)) == -4
    assert L.kvq_decode_step(*s_args(FAKE, 255)) == -4
    assert L.kvq_decode_step(*s_args(FAKE, -2)) == -1
    assert L.kvq_decode_step(*s_args(FAKE, 256, ws=16)) == -6
    # allocation-free decode: the decode checks, and a plan whose partials exceed the
    # library's fixed array is refused (KVQ_ERR_WORKSPACE) before any HIP call
    n_args = lambda nq, max_len, n_seq=1, q=FAKE, out=FAKE: (C.byref(good), nq, q, FAKE, FAKE, FAKE, n_seq, max_len,
                                                             FAKE, FAKE, FAKE, 0.1, out, None)
    assert L.kvq_packed_decode_attn_noalloc(*n_args(3, 512)) == -2
    assert L.kvq_packed_decode_attn_noalloc(*n_args(16, 2048)) == -5
    assert L.kvq_packed_decode_attn_noalloc(*n_args(16, 512, q=FAKE + 8)) == -4
    assert L.kvq_packed_decode_attn_noalloc(*n_args(16, 512, out=None)) == -1
    assert kvq.decode_workspace_bytes(good, 16, 60000, 512) > kvq.NOALLOC_SCRATCH_BYTES
    assert L.kvq_packed_decode_attn_noalloc(*n_args(16, 512, n_seq=60000)) == -6
    assert L.kvq_packed_decode_attn_noalloc(*n_args(16, 512, n_seq=0)) == 0  # nothing to do
    # fp16 window: window range, ring and new-row alignment, workspace, before any HIP call
    w_args = lambda win, wk, kn, ss, ws=1 << 30: (C.byref(good), win, 16, FAKE, kn, FAKE, ss, 128, wk, FAKE, FAKE, FAKE,
                                                  FAKE, 1, 512, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, ws, 0, 0, None)
    assert L.kvq_window_decode_step(*w_args(0, FAKE, FAKE, 256)) == -1
    assert L.kvq_window_decode_step(*w_args(1025, FAKE, FAKE, 256)) == -1
    assert L.kvq_window_decode_step(*w_args(64, None, FAKE, 256)) == -1
    assert L.kvq_window_decode_step(*w_args(64, FAKE + 4, FAKE, 256)) == -4
    assert L.kvq_window_decode_step(*w_args(64, FAKE, None, 256)) == -1
    assert L.kvq_window_decode_step(*w_args(64, FAKE, FAKE + 4, 256)) == -4
    assert L.kvq_window_decode_step(*w_args(64, FAKE, FAKE, 260)) == -4
    assert L.kvq_window_decode_step(*w_args(64, FAKE, FAKE, 256, ws=16)) == -6
    a_args = lambda win, wk, ws=1 << 30: (C.byref(good), win, 16, FAKE, wk, FAKE, FAKE, FAKE, FAKE, 1, 512, FAKE,
                                          FAKE, FAKE, 0.1, FAKE, FAKE, ws, 0, 0, None)
    assert L.kvq_window_decode_attn(*a_args(2000, FAKE)) == -1
    assert L.kvq_window_decode_attn(*a_args(64, FAKE + 8)) == -4
    assert L.kvq_window_decode_attn(*a_args(64, FAKE, ws=16)) == -6
    # chunked prefill: served geometries, capacity, pointers, alignment, workspace
    p_args = lambda g_, nq, max_len, ws, q=FAKE, n_split=4, wsp=FAKE: (
        C.byref(g_), nq, q, FAKE, FAKE, FAKE, FAKE, 1, 64, max_len, FAKE, FAKE, FAKE, 0.1, FAKE, wsp, ws, n_split,
        None)
    assert kvq.prefill_plan(good, 16, 1, 64, 512, 4) == {"n_split": 4, "workspace": 64 * 16 * 4 * 130 * 4}
    assert kvq.prefill_workspace_bytes(good, 16, 1, 64, 512, 1) == 0
    assert L.kvq_packed_prefill_attn(*p_args(good, 3, 512, 1 << 30)) == -2           # GQA ratio
    assert L.kvq_packed_prefill_attn(*p_args(good, 2 * 129, 512, 1 << 30)) == -2     # group > 128
    # passthrough widths (K16, the K-only V16) are served
    assert kvq.prefill_plan(kvq.geom(2, 1024, 16, 1024), 16, 1, 64, 512, 1)["n_split"] == 1
    assert kvq.prefill_plan(kvq.geom(2, 192, 16, 1024), 16, 1, 64, 512, 2)["n_split"] == 2
    assert L.kvq_packed_prefill_attn(*p_args(kvq.geom(2, 192, 3, 1024, head_dim=64), 16, 512, 1 << 30)) == -2
    assert L.kvq_packed_prefill_attn(*p_args(good, 16, 2048, 1 << 30)) == -5
    assert L.kvq_packed_prefill_attn(*p_args(good, 16, 512, 16)) == -6
    assert L.kvq_packed_prefill_attn(*p_args(good, 16, 512, 1 << 30, q=FAKE + 8)) == -4
    assert L.kvq_packed_prefill_attn(*p_args(good, 16, 512, 1 << 30, q=None)) == -1
    assert L.kvq_packed_prefill_attn(*p_args(good, 16, 512, 1 << 30, wsp=None)) == -1
    assert L.kvq_packed_prefill_attn(*p_args(good, 16, 512, 1 << 30, n_split=-1)) == -1
    # rotated variant: uniform key widths 1..8 (k_budget a multiple of 64), v_bits <= 8,
    # pointers, alignment, capacity, GQA ratio -- all before any HIP call
    r_args = lambda g_, max_new=4, k=FAKE, vsg=FAKE, vsig=FAKE: (
        C.byref(g_), k, FAKE, 256, 128, 1, FAKE, FAKE, FAKE, max_new, FAKE, vsg, vsig, FAKE, FAKE, None)
    assert L.kvq_rot_quantize_pack(*r_args(kvq.geom(2, 160, 3, 1024))) == -3
    assert L.kvq_rot_quantize_pack(*r_args(kvq.geom(2, 192, 16, 1024))) == -3
    assert L.kvq_rot_quantize_pack(*r_args(kvq.geom(2, 0, 3, 1024))) == -3
    assert L.kvq_rot_quantize_pack(*r_args(good, max_new=2048)) == -5
    assert L.kvq_rot_quantize_pack(*r_args(good, k=None)) == -1
    assert L.kvq_rot_quantize_pack(*r_args(good, vsg=None, vsig=None)) == -1
    assert L.kvq_rot_quantize_pack(*r_args(good, k=FAKE + 2)) == -4
    assert L.kvq_rot_quantize_pack(*r_args(good, max_new=0)) == 0  # nothing to do
    assert L.kvq_rot_queries(C.byref(good), 3, 1, FAKE, FAKE, FAKE, None) == -2
    assert L.kvq_rot_queries(C.byref(good), 16, 1, FAKE, None, FAKE, None) == -1
    assert L.kvq_rot_queries(C.byref(good), 16, 1, FAKE + 2, FAKE, FAKE, None) == -4
    assert L.kvq_rot_queries(C.byref(kvq.geom(2, 100, 3, 1024)), 16, 1, FAKE, FAKE, FAKE, None) == -3
    assert L.kvq_rot_queries(C.byref(good), 16, 0, FAKE, FAKE, FAKE, None) == 0
    assert L.kvq_rot_back(C.byref(good), 16, 1, FAKE + 4, FAKE, None) == -4
    assert L.kvq_rot_back(C.byref(good), 16, 1, FAKE, None, None) == -1
    assert L.kvq_rot_back(C.byref(good), 16, -1, FAKE, FAKE, None) == -1
    assert L.kvq_rot_back(C.byref(kvq.geom(2, 192, 16, 1024)), 16, 1, FAKE, FAKE, None) == -3
    rp = lambda g_, nq=16, q=FAKE, kn=FAKE, ss=256, vsg=FAKE, vsig=FAKE: (
        C.byref(g_), nq, 1, q, FAKE, kn, FAKE, ss, 128, FAKE, FAKE, FAKE, FAKE, vsg, vsig, None)
    assert L.kvq_rot_decode_prepare(*rp(kvq.geom(2, 160, 3, 1024))) == -3
    assert L.kvq_rot_decode_prepare(*rp(good, nq=3)) == -2
    assert L.kvq_rot_decode_prepare(*rp(good, q=None)) == -1
    assert L.kvq_rot_decode_prepare(*rp(good, vsg=None, vsig=None)) == -1
    assert L.kvq_rot_decode_prepare(*rp(good, kn=FAKE + 2)) == -4
    assert L.kvq_rot_decode_prepare(*rp(good, ss=255)) == -4
    rs = lambda g_, nq=16, q=FAKE, kn=FAKE, ss=256, ksg=FAKE, nb=1 << 30, ml=1024: (
        C.byref(g_), nq, q, kn, FAKE, ss, 128, FAKE, FAKE, FAKE, 1, ml, FAKE, FAKE, FAKE, ksg, FAKE, 0.088, FAKE, nb,
        0, None)
    assert L.kvq_rot_decode_step_partials(*rs(kvq.geom(2, 160, 3, 1024))) == -3   # rotated keys: uniform widths
    assert L.kvq_rot_decode_step_partials(*rs(kvq.geom(2, 320, 3, 1024))) == -2   # K record past the MFMA kernel's
    assert L.kvq_rot_decode_step_partials(*rs(good, nq=3)) == -2
    assert L.kvq_rot_decode_step_partials(*rs(good, q=None)) == -1
    assert L.kvq_rot_decode_step_partials(*rs(good, ksg=None)) == -1
    assert L.kvq_rot_decode_step_partials(*rs(good, kn=FAKE + 2)) == -4
    assert L.kvq_rot_decode_step_partials(*rs(good, ss=255)) == -4
    assert L.kvq_rot_decode_step_partials(*rs(good, nb=16)) == -6
    assert L.kvq_rot_decode_step_partials(*rs(good, ml=4096)) == -5
    # read probe (measurement helper): counts, pointers, alignment
    assert L.kvq_read_probe(FAKE, -16, FAKE, 4, None) == -1
    assert L.kvq_read_probe(FAKE, 1024, FAKE, 0, None) == -1
    assert L.kvq_read_probe(None, 1024, FAKE, 4, None) == -1
    assert L.kvq_read_probe(FAKE + 4, 1024, FAKE, 4, None) == -4
    assert L.kvq_read_probe(FAKE, 1000, FAKE, 4, None) == -4
    assert L.kvq_read_probe(FAKE, 0, FAKE, 4, None) == 0
