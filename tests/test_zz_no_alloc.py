"""The allocation-free decode entry point (kvq_packed_decode_attn_noalloc) against
kvq_packed_decode_attn, through the C ABI: two calls in a row on the same GPU, the
second with a smaller batch and shorter sequences, each equal to the workspace
call's output and within 2e-3 of the oracle's exact attention."""
import numpy as np
import pytest
import torch

import oracle
from packed_cache_attention_amd import kvq, synth

from pipeline import check_attention, run_batch, say

pytestmark = pytest.mark.gpu


def _case(lens, seed, wl=None):
    wl = wl or synth.WORKLOADS["c3"]
    seqs = []
    for i, n in enumerate(lens):
        K, V, q = synth.gen_layer(wl, i, 0, n_tok=n, seed=seed)
        seqs.append((K, V, q))
    cap = synth.ceil_to(max(lens), 64) + 64
    return run_batch(seqs, wl.k_budget, wl.v_bits, cap, check_attn=False), seqs


def _compare(lens, seed, wl=None):
    say("noalloc: lens %s seed %d %s" % (list(lens), seed, wl.name if wl else "c3"))
    res, seqs = _case(lens, seed, wl)
    g, cache, off = res["g"], res["cache"], res["off"]
    n_seq, n_q = len(lens), seqs[0][2].shape[0]
    q = torch.stack([s[2] for s in seqs], 0).cuda().contiguous()
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    max_len = max(lens)
    need = kvq.decode_workspace_bytes(g, n_q, n_seq, max_len)
    assert need <= kvq.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need // 4 + 4, dtype=torch.float32, device="cuda")
    ref_out = torch.empty(n_seq, n_q, 128, dtype=torch.float32, device="cuda")
    kvq.packed_decode_attn(g, q, cache, off, seq_len, max_len, res["kbits"], res["ksig"], res["vsig"], ref_out, ws)
    out = torch.full((n_seq, n_q, 128), float("nan"), dtype=torch.float32, device="cuda")
    kvq.packed_decode_attn_noalloc(g, q, cache, off, seq_len, max_len, res["kbits"], res["ksig"], res["vsig"], out)
    torch.cuda.synchronize()
    a, b = out.cpu().numpy(), ref_out.cpu().numpy()
    # the same kernels and plan: identical bits
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    region = kvq.cache_bytes(g)
    ref = np.stack([oracle.decode_attention(res["ogeom"], res["oc"][i * region:(i + 1) * region],
                                            seqs[i][2].numpy(), lens[i], res["ob"], res["osig"], res["ovsig"])
                    for i in range(n_seq)])
    say("noalloc: worst relative error %.2e" % check_attention(a, ref))


def test_noalloc_two_calls_second_smaller():
    """The second call reuses the array the first filled with more partials."""
    _compare((2100, 777, 64, 1), seed=3)
    _compare((900, 130), seed=4)


def test_noalloc_generic_kernel():
    """Geometries the vector-ALU kernel serves (its query table then lives in the array
    too): K records over 64 bytes (K16 with 16-bit values) and a GQA group of 12."""
    import dataclasses
    base = synth.WORKLOADS["c3"]
    k16 = dataclasses.replace(base, name="k16v16", k_budget=1024, v_bits=16)
    g12 = dataclasses.replace(base, name="group12", n_q_heads=12, n_kv_heads=1)
    for wl in (k16, g12):
        g = kvq.geom(wl.n_kv_heads, wl.k_budget, wl.v_bits, 1024)
        assert kvq.decode_plan(g, wl.n_q_heads, 2, 1024)["kernel"] == kvq.DECODE_GENERIC
        _compare((700, 64), seed=5, wl=wl)
        _compare((130,), seed=6, wl=wl)


def test_noalloc_konly_values():
    """The K-only value mode (16-bit values) on the matrix-core kernel."""
    import dataclasses
    konly = dataclasses.replace(synth.WORKLOADS["c3"], name="konly", v_bits=16)
    g = kvq.geom(konly.n_kv_heads, konly.k_budget, konly.v_bits, 1024)
    assert kvq.decode_plan(g, konly.n_q_heads, 2, 1024)["kernel"] == kvq.DECODE_MFMA
    _compare((700, 64), seed=7, wl=konly)
    _compare((130,), seed=8, wl=konly)


def test_noalloc_rejects_plan_beyond_the_array():
    g = kvq.geom(2, 192, 3, 1024)
    n_seq = 60000
    assert kvq.decode_workspace_bytes(g, 16, n_seq, 512) > kvq.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(n_seq, 16, 128, dtype=torch.float16, device="cuda")
    out = torch.zeros(n_seq, 16, 128, dtype=torch.float32, device="cuda")
    z = torch.zeros(n_seq, dtype=torch.int64, device="cuda")
    lens = torch.zeros(n_seq, dtype=torch.int32, device="cuda")
    small = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.packed_decode_attn_noalloc(g, q, small, z, lens, 512, small, small.float(), small.float(), out)
    assert e.value.status == -6
