"""GPU parity of the rotated (TurboQuant-MSE proper) variant against the oracle.

Page: "RoPE-Aware Bit Allocation for KV-Cache Quantization", abstract -- Block-GTQ is
built on TurboQuant-MSE, whose base step rotates each key by a random-sign
Walsh-Hadamard transform and codes every rotated coordinate with the Gaussian
Lloyd-Max codebook at one uniform width (the related-papers page for "Quantization
Dominates Rank Reduction for KV-Cache" names its key path "WHT + MSE").

Compared: the packed cache bytes of kvq_rot_quantize_pack (bit-exact, one call for a
ragged batch, then a ragged append into partly filled tiles), the rotated queries of
kvq_rot_queries (bit-exact), and decode attention over the rotated cache --
kvq_rot_queries, kvq_packed_decode_attn with uniform widths and the rotation scale,
then kvq_rot_back -- against the oracle's exact attention of the same method, within
the attention tolerance.  Values are rotated (their own signs) or coded unrotated with
per-block scales; both RoPE pairings."""
import numpy as np
import pytest
import torch

import oracle
from packed_cache_attention_amd import kvq, synth

from pipeline import check_attention, say

pytestmark = pytest.mark.gpu

D = 128
SIG_ROT = np.array([0x3DB504F3], np.uint32).view(np.float32)[0]


def _batch(H, grp, kb, vb, lens, seed, layer=0):
    wl = synth.Workload("rot", 1, H * grp, H, 1e6, (0,), kb, vb, "decay")
    return [synth.gen_layer(wl.with_lens([n]), i, layer, n_tok=n, seed=seed) for i, n in enumerate(lens)]


def _gpu_pack(g, seqs, first, ksg, vsg, vsig, cache, off):
    lens = [s[0].shape[0] for s in seqs]
    rows = torch.cat([s[0] for s in seqs], 0).cuda()
    vrows = torch.cat([s[1] for s in seqs], 0).cuda()
    row0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    kvq.rot_quantize_pack(g, rows, vrows, torch.tensor(first, dtype=torch.int64, device="cuda"),
                          torch.tensor(lens, dtype=torch.int32, device="cuda"),
                          torch.tensor(row0, dtype=torch.int64, device="cuda"), max(lens), ksg.cuda(),
                          None if vsg is None else vsg.cuda(), None if vsig is None else torch.from_numpy(vsig).cuda(),
                          cache, off)


def _oracle_pack(ogeom, oc, seqs, first, ksg, vsg, vsig):
    region = ogeom.seq_bytes
    for i, (K, V, _) in enumerate(seqs):
        if K.shape[0]:
            oracle.quantize_pack_rot(ogeom, oc[i * region:(i + 1) * region], K.numpy(), V.numpy(), first[i],
                                     ksg.numpy(), None if vsg is None else vsg.numpy(), vsig)


def _check_bytes(cache, oc, what):
    gc = cache.cpu().numpy()
    if not np.array_equal(gc, oc):
        bad = np.nonzero(gc != oc)[0]
        raise AssertionError("%s: packed bytes differ at %d positions, first %s" % (what, len(bad), bad[:8]))


def _run(H, grp, kb, vb, pairing, vrot, lens, extra, cap, kernel=kvq.DECODE_AUTO, tiles=0, seed=3, qscale=1.0):
    """Pack `lens` tokens per sequence, append `extra` more, decode; returns worst rel error."""
    say("rotation: H %d g %d kb %d vb %d pairing %d vrot %d lens %s extra %s kernel %d tiles %d"
        % (H, grp, kb, vb, pairing, vrot, lens, extra, kernel, tiles))
    full = [n + e for n, e in zip(lens, extra)]
    seqs = _batch(H, grp, kb, vb, full, seed)
    ksg = synth.rot_signs(H, seed=seed)
    vsg = synth.rot_signs(H, seed=seed + 1) if vrot else None
    vsig = None
    if not vrot:
        ev = np.zeros((H, D // 2, 2), np.uint64)
        for _, V, _ in seqs:
            oracle.block_energy(V.numpy(), pairing, ev)
        _, vsig = oracle.allocate(ev, vb * (D // 2), oracle.UNIFORM)
    g = kvq.geom(H, kb, vb, cap, rope_pairing=pairing)
    ogeom = oracle.Geometry(H, kb, vb, cap, pairing=pairing)
    region = kvq.cache_bytes(g)
    assert region == ogeom.seq_bytes
    nseq = len(seqs)
    cache = torch.zeros(nseq * region, dtype=torch.uint8, device="cuda")
    off = torch.arange(nseq, dtype=torch.int64, device="cuda") * region
    oc = np.zeros(nseq * region, np.uint8)
    head = [(K[:n], V[:n], q) for (K, V, q), n in zip(seqs, lens)]
    _gpu_pack(g, head, [0] * nseq, ksg, vsg, vsig, cache, off)
    _oracle_pack(ogeom, oc, head, [0] * nseq, ksg, vsg, vsig)
    _check_bytes(cache, oc, "first call")
    if any(extra):
        tail = [(K[n:], V[n:], q) for (K, V, q), n in zip(seqs, lens)]
        _gpu_pack(g, tail, list(lens), ksg, vsg, vsig, cache, off)
        _oracle_pack(ogeom, oc, tail, list(lens), ksg, vsg, vsig)
        _check_bytes(cache, oc, "append")
    # queries rotated once
    q = torch.stack([(s[2].float() * qscale).half() for s in seqs], 0).cuda().contiguous()
    q_rot = torch.empty_like(q)
    kvq.rot_queries(g, q, q_rot, ksg.cuda())
    qc, qr = q.cpu().numpy(), q_rot.cpu().numpy().view(np.uint16)
    for i in range(nseq):
        for h in range(H * grp):
            np.testing.assert_array_equal(qr[i, h], oracle.rot_query(qc[i, h], ksg[h // grp].numpy()))
    # attention over the rotated cache, then the output rotated back
    seq_len = torch.tensor(full, dtype=torch.int32, device="cuda")
    max_len = max(full)
    kbits = torch.full((H, D // 2), kb // (D // 2), dtype=torch.uint8, device="cuda")
    ksig = torch.full((H, D // 2), float(SIG_ROT), dtype=torch.float32, device="cuda")
    vs = ksig if vrot else torch.from_numpy(vsig).cuda()
    ws = torch.empty(kvq.decode_workspace_bytes(g, H * grp, nseq, max_len, kernel, tiles) // 4 + 4,
                     dtype=torch.float32, device="cuda")
    out = torch.empty(nseq, H * grp, D, dtype=torch.float32, device="cuda")
    kvq.packed_decode_attn(g, q_rot, cache, off, seq_len, max_len, kbits, ksig, vs, out, ws, kernel=kernel,
                           tiles_per_split=tiles)
    if vrot:
        kvq.rot_back(g, out, vsg.cuda())
    o = out.cpu().numpy()
    ref = np.stack([oracle.decode_attention_rot(ogeom, oc[i * region:(i + 1) * region], qc[i], full[i],
                                                ksg.numpy(), None if vsg is None else vsg.numpy(), vsig)
                    for i in range(nseq)])
    worst = check_attention(o, ref)
    say("worst rel %.2e" % worst)
    return worst


@pytest.mark.parametrize("vrot", [True, False], ids=["vrot", "vplain"])
@pytest.mark.parametrize("pairing", [kvq.PAIR_HALF, kvq.PAIR_INTERLEAVED], ids=["half", "interleaved"])
@pytest.mark.parametrize("geom", [(2, 8, 192, 3), (2, 4, 128, 2), (1, 7, 64, 1), (3, 2, 256, 4)],
                         ids=["k3v3g8", "k2v2g4", "k1v1g7", "k4v4g2"])
def test_rotated_pack_and_decode(geom, pairing, vrot):
    H, grp, kb, vb = geom
    _run(H, grp, kb, vb, pairing, vrot, lens=(1000, 333, 64, 1), extra=(5, 64, 0, 130), cap=1152)


@pytest.mark.parametrize("kernel", [kvq.DECODE_AUTO, kvq.DECODE_GENERIC])
@pytest.mark.parametrize("vb", [8, 5])
def test_rotated_widest(kernel, vb):
    """Width 8 everywhere (records of 128 bytes: the generic kernel serves them)."""
    _run(2, 4, 512, vb, kvq.PAIR_HALF, True, lens=(700, 70), extra=(1, 63), cap=832, kernel=kernel)


@pytest.mark.parametrize("tiles", [1, 3])
def test_rotated_split_plans(tiles):
    _run(2, 8, 192, 3, kvq.PAIR_HALF, True, lens=(1000, 129, 640), extra=(24, 0, 1), cap=1088, tiles=tiles,
         kernel=kvq.DECODE_MFMA)


def test_rotated_queries_large_and_tiny():
    """Queries of magnitude 10^-6 .. 10^2 (still fitting binary16 once rotated)."""
    _run(2, 8, 192, 3, kvq.PAIR_HALF, True, lens=(300,), extra=(0,), cap=320, qscale=100.0)
    _run(2, 8, 192, 3, kvq.PAIR_HALF, True, lens=(300,), extra=(0,), cap=320, qscale=1e-6)


def test_rotated_c3_layer_full_size():
    """One 128K-token Qwen2.5-3B-shaped layer (2 KV heads, 16 query heads, K3V3) through
    the rotated path in the automatic plan the decode kernel is timed in."""
    wl = synth.WORKLOADS["c3"]
    n = wl.seq_lens[0]
    _run(wl.n_kv_heads, wl.group, wl.k_budget, wl.v_bits, kvq.PAIR_HALF, True, lens=(n - 1,), extra=(1,),
         cap=synth.ceil_to(n + 64, 64), seed=7)


@pytest.mark.parametrize("vrot", [True, False], ids=["vrot", "vplain"])
@pytest.mark.parametrize("pairing", [kvq.PAIR_HALF, kvq.PAIR_INTERLEAVED], ids=["half", "interleaved"])
@pytest.mark.parametrize("kb,vb", [(192, 3), (512, 8), (64, 1)], ids=["k3v3", "k8v8", "k1v1"])
def test_rotated_decode_prepare(kb, vb, pairing, vrot):
    """kvq_rot_decode_prepare: the new token of each sequence packed at slot seq_len - 1
    (bytes equal to the oracle's packing of every token; lengths 0, 63, 64, 127 and 300
    before the step, so the token opens a tile, fills one, or lands mid-tile) and the
    queries rotated (bits equal to the oracle's), then attention within 2e-3."""
    H, grp = 2, 4
    lens = [0, 63, 64, 127, 300]
    say("rot prepare: kb %d vb %d pairing %d vrot %d" % (kb, vb, pairing, vrot))
    seqs = _batch(H, grp, kb, vb, [n + 1 for n in lens], seed=31)
    ksg = synth.rot_signs(H, seed=31)
    vsg = synth.rot_signs(H, seed=32) if vrot else None
    vsig = None
    if not vrot:
        ev = np.zeros((H, D // 2, 2), np.uint64)
        for _, V, _ in seqs:
            oracle.block_energy(V.numpy(), pairing, ev)
        _, vsig = oracle.allocate(ev, vb * (D // 2), oracle.UNIFORM)
    cap = 384
    g = kvq.geom(H, kb, vb, cap, rope_pairing=pairing)
    ogeom = oracle.Geometry(H, kb, vb, cap, pairing=pairing)
    region = kvq.cache_bytes(g)
    S = len(lens)
    cache = torch.zeros(S * region, dtype=torch.uint8, device="cuda")
    off = torch.arange(S, dtype=torch.int64, device="cuda") * region
    head = [(K[:n], V[:n], q) for (K, V, q), n in zip(seqs, lens) if n > 0]
    idx = [i for i, n in enumerate(lens) if n > 0]
    # the prefill (sequences with tokens), one call
    rows = torch.cat([x[0] for x in head], 0).cuda()
    vrows = torch.cat([x[1] for x in head], 0).cuda()
    first = torch.zeros(S, dtype=torch.int64, device="cuda")
    nn = torch.tensor(lens, dtype=torch.int32, device="cuda")
    row0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    kvq.rot_quantize_pack(g, rows, vrows, first, nn, torch.tensor(row0, device="cuda"),
                          max(lens), ksg.cuda(), None if vsg is None else vsg.cuda(),
                          None if vsig is None else torch.from_numpy(vsig).cuda(), cache, off)
    # the step: new tokens and queries
    kn = torch.stack([K[n] for (K, _, _), n in zip(seqs, lens)]).cuda()
    vn = torch.stack([V[n] for (_, V, _), n in zip(seqs, lens)]).cuda()
    q = torch.stack([x[2] for x in seqs]).cuda().contiguous()
    q_rot = torch.empty_like(q)
    seq_len = torch.tensor([n + 1 for n in lens], dtype=torch.int32, device="cuda")
    kvq.rot_decode_prepare(g, q, q_rot, kn, vn, cache, off, seq_len, ksg.cuda(), None if vsg is None else vsg.cuda(),
                           None if vsig is None else torch.from_numpy(vsig).cuda())
    oc = np.zeros(S * region, np.uint8)
    for i, (K, V, _) in enumerate(seqs):
        oracle.quantize_pack_rot(ogeom, oc[i * region:(i + 1) * region], K.numpy(), V.numpy(), 0, ksg.numpy(),
                                 None if vsg is None else vsg.numpy(), vsig)
    _check_bytes(cache, oc, "prepare")
    qc, qr = q.cpu().numpy(), q_rot.cpu().numpy().view(np.uint16)
    for i in range(S):
        for h in range(H * grp):
            np.testing.assert_array_equal(qr[i, h], oracle.rot_query(qc[i, h], ksg[h // grp].numpy()))
    kbits = torch.full((H, D // 2), kb // (D // 2), dtype=torch.uint8, device="cuda")
    ksig = torch.full((H, D // 2), float(SIG_ROT), dtype=torch.float32, device="cuda")
    vs = ksig if vrot else torch.from_numpy(vsig).cuda()
    ws = torch.empty(kvq.decode_workspace_bytes(g, H * grp, S, cap) // 4 + 4, dtype=torch.float32, device="cuda")
    out = torch.empty(S, H * grp, D, dtype=torch.float32, device="cuda")
    kvq.packed_decode_attn(g, q_rot, cache, off, seq_len, cap, kbits, ksig, vs, out, ws)
    if vrot:
        kvq.rot_back(g, out, vsg.cuda())
    ref = np.stack([oracle.decode_attention_rot(ogeom, oc[i * region:(i + 1) * region], qc[i], lens[i] + 1,
                                                ksg.numpy(), None if vsg is None else vsg.numpy(), vsig)
                    for i in range(S)])
    say("worst rel %.2e" % check_attention(out.cpu().numpy(), ref))


@pytest.mark.parametrize("tiles", [0, 1])
@pytest.mark.parametrize("vrot", [True, False], ids=["vrot", "vplain"])
@pytest.mark.parametrize("pairing", [kvq.PAIR_HALF, kvq.PAIR_INTERLEAVED], ids=["half", "interleaved"])
@pytest.mark.parametrize("kb,vb", [(192, 3), (64, 1), (256, 4), (128, 8)], ids=["k3v3", "k1v1", "k4v4", "k2v8"])
def test_rotated_fused_step(kb, vb, pairing, vrot, tiles):
    """kvq_rot_decode_step_partials (queries and the new token rotated inside the
    attention kernel) against kvq_rot_decode_prepare + kvq_decode_partials on the rotated
    queries: the same cache bytes (and so the oracle's), the same partials bit for bit,
    then merged (and rotated back) within 2e-3 of the oracle.  Lengths 0, 63, 64, 127 and
    300 before the step; one tile per chunk or the planner's chunks."""
    H, grp = 2, 4
    lens = [0, 63, 64, 127, 300]
    say("rot fused step: kb %d vb %d pairing %d vrot %d tiles %d" % (kb, vb, pairing, vrot, tiles))
    seqs = _batch(H, grp, kb, vb, [n + 1 for n in lens], seed=51)
    ksg = synth.rot_signs(H, seed=51).cuda()
    vsg = synth.rot_signs(H, seed=52).cuda() if vrot else None
    vsig = None
    if not vrot:
        ev = np.zeros((H, D // 2, 2), np.uint64)
        for _, V, _ in seqs:
            oracle.block_energy(V.numpy(), pairing, ev)
        _, vsig = oracle.allocate(ev, vb * (D // 2), oracle.UNIFORM)
    cap = 384
    g = kvq.geom(H, kb, vb, cap, rope_pairing=pairing)
    ogeom = oracle.Geometry(H, kb, vb, cap, pairing=pairing)
    region = kvq.cache_bytes(g)
    S = len(lens)
    cache = torch.zeros(S * region, dtype=torch.uint8, device="cuda")
    off = torch.arange(S, dtype=torch.int64, device="cuda") * region
    head = [(K[:n], V[:n], q) for (K, V, q), n in zip(seqs, lens) if n > 0]
    rows = torch.cat([x[0] for x in head], 0).cuda()
    vrows = torch.cat([x[1] for x in head], 0).cuda()
    row0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    vsig_t = None if vsig is None else torch.from_numpy(vsig).cuda()
    kvq.rot_quantize_pack(g, rows, vrows, torch.zeros(S, dtype=torch.int64, device="cuda"),
                          torch.tensor(lens, dtype=torch.int32, device="cuda"), torch.tensor(row0, device="cuda"),
                          max(lens), ksg, vsg, vsig_t, cache, off)
    kn = torch.stack([K[n] for (K, _, _), n in zip(seqs, lens)]).cuda()
    vn = torch.stack([V[n] for (_, V, _), n in zip(seqs, lens)]).cuda()
    q = torch.stack([x[2] for x in seqs]).cuda().contiguous()
    seq_len = torch.tensor([n + 1 for n in lens], dtype=torch.int32, device="cuda")
    kbits = torch.full((H, D // 2), kb // (D // 2), dtype=torch.uint8, device="cuda")
    ksig = torch.full((H, D // 2), float(SIG_ROT), dtype=torch.float32, device="cuda")
    vs = ksig if vrot else vsig_t
    plan = kvq.decode_plan(g, H * grp, S, cap, kvq.DECODE_MFMA, tiles)
    part_a = torch.full((plan["workspace"] // 4,), float("nan"), dtype=torch.float32, device="cuda")
    part_b = part_a.clone()
    cache_b = cache.clone()
    # two launches: the step's preparation, then the split phase on the rotated queries
    q_rot = torch.empty_like(q)
    kvq.rot_decode_prepare(g, q, q_rot, kn, vn, cache, off, seq_len, ksg, vsg, vsig_t)
    kvq.decode_partials(g, q_rot, cache, off, seq_len, cap, kbits, ksig, vs, part_a, kernel=kvq.DECODE_MFMA,
                        tiles_per_split=tiles)
    # one launch
    kvq.rot_decode_step_partials(g, q, kn, vn, cache_b, off, seq_len, cap, kbits, ksig, vs, ksg, vsg, part_b,
                                 tiles_per_split=tiles)
    np.testing.assert_array_equal(cache_b.cpu().numpy(), cache.cpu().numpy())
    oc = np.zeros(S * region, np.uint8)
    for i, (K, V, _) in enumerate(seqs):
        oracle.quantize_pack_rot(ogeom, oc[i * region:(i + 1) * region], K.numpy(), V.numpy(), 0, ksg.cpu().numpy(),
                                 None if vsg is None else vsg.cpu().numpy(), vsig)
    _check_bytes(cache_b, oc, "fused step")
    ns = plan["n_split"]
    pa = part_a[:S * H * grp * ns * 130].view(S * H * grp, ns, 130).cpu().numpy()
    pb = part_b[:S * H * grp * ns * 130].view(S * H * grp, ns, 130).cpu().numpy()
    np.testing.assert_array_equal(pb.view(np.uint32), pa.view(np.uint32))
    out = torch.empty(S, H * grp, D, dtype=torch.float32, device="cuda")
    kvq.merge_partials(S, H * grp, ns, part_b, out)
    if vrot:
        kvq.rot_back(g, out, vsg)
    ref = np.stack([oracle.decode_attention_rot(ogeom, oc[i * region:(i + 1) * region], q.cpu().numpy()[i],
                                                lens[i] + 1, ksg.cpu().numpy(),
                                                None if vsg is None else vsg.cpu().numpy(), vsig)
                    for i in range(S)])
    say("worst rel %.2e" % check_attention(out.cpu().numpy(), ref))


def test_rotated_fused_step_full_size():
    """The rotated step as the bench times it, at its size: one 128K-token Qwen2.5-3B-shaped
    layer (K3V3, values rotated), the 131073rd token appended by kvq_rot_decode_step_partials
    in the automatic plan with max_len = capacity; the cache bytes against the oracle's
    rotated packing of all tokens, the merged and back-rotated output within 2e-3 of the
    oracle's attention over them."""
    wl = synth.WORKLOADS["c3"]
    H, grp, kb, vb = wl.n_kv_heads, wl.group, wl.k_budget, wl.v_bits
    n = wl.seq_lens[0]
    say("rot fused step full size: %d tokens" % n)
    (K, V, q), = _batch(H, grp, kb, vb, [n + 1], seed=13)
    ksg, vsg = synth.rot_signs(H, seed=13), synth.rot_signs(H, seed=14)
    cap = synth.ceil_to(n + 64, 64)
    g = kvq.geom(H, kb, vb, cap)
    ogeom = oracle.Geometry(H, kb, vb, cap)
    cache = torch.zeros(kvq.cache_bytes(g), dtype=torch.uint8, device="cuda")
    off = torch.zeros(1, dtype=torch.int64, device="cuda")
    _gpu_pack(g, [(K[:n], V[:n], q)], [0], ksg, vsg, None, cache, off)
    kbits = torch.full((H, D // 2), kb // (D // 2), dtype=torch.uint8, device="cuda")
    sig = torch.full((H, D // 2), float(SIG_ROT), dtype=torch.float32, device="cuda")
    plan = kvq.decode_plan(g, H * grp, 1, cap)
    say("plan %s" % plan)
    assert plan["kernel"] == kvq.DECODE_MFMA
    part = torch.empty(plan["workspace"] // 4 + 4, dtype=torch.float32, device="cuda")
    seq_len = torch.tensor([n + 1], dtype=torch.int32, device="cuda")
    kvq.rot_decode_step_partials(g, q[None].cuda().contiguous(), K[n:n + 1].cuda().contiguous(),
                                 V[n:n + 1].cuda().contiguous(), cache, off, seq_len, cap, kbits, sig, sig,
                                 ksg.cuda(), vsg.cuda(), part)
    out = torch.empty(1, H * grp, D, dtype=torch.float32, device="cuda")
    kvq.merge_partials(1, H * grp, plan["n_split"], part, out)
    kvq.rot_back(g, out, vsg.cuda())
    oc = np.zeros(kvq.cache_bytes(g), np.uint8)
    _oracle_pack(ogeom, oc, [(K, V, q)], [0], ksg, vsg, None)
    _check_bytes(cache, oc, "fused step, full size")
    ref = oracle.decode_attention_rot(ogeom, oc, q.numpy(), n + 1, ksg.numpy(), vsg.numpy(), None)
    say("worst rel %.2e" % check_attention(out.cpu().numpy()[0], ref))


def test_rotated_fused_step_rejects_wide_keys():
    """Rotated keys wider than 4 bits (K records over 64 bytes) have no matrix-core step:
    the fused call reports KVQ_ERR_SHAPE and writes nothing."""
    H, grp, kb, vb, cap = 2, 4, 320, 3, 128
    g = kvq.geom(H, kb, vb, cap)
    cache = torch.zeros(kvq.cache_bytes(g), dtype=torch.uint8, device="cuda")
    z = torch.zeros(1, dtype=torch.int64, device="cuda")
    x = torch.zeros(1, H, D, dtype=torch.float16, device="cuda")
    q = torch.zeros(1, H * grp, D, dtype=torch.float16, device="cuda")
    sg = torch.zeros(H, D, dtype=torch.uint8, device="cuda")
    kbits = torch.full((H, D // 2), kb // (D // 2), dtype=torch.uint8, device="cuda")
    sig = torch.full((H, D // 2), float(SIG_ROT), dtype=torch.float32, device="cuda")
    part = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError) as err:
        kvq.rot_decode_step_partials(g, q, x, x, cache, z, torch.ones(1, dtype=torch.int32, device="cuda"), cap,
                                     kbits, sig, sig, sg, sg, part)
    assert err.value.status == -2
    torch.cuda.synchronize()
    assert int(cache.count_nonzero()) == 0


@pytest.mark.parametrize("align", ["4byte", "16byte-oddstride"])
@pytest.mark.parametrize("vrot", [True, False], ids=["vrot", "vplain"])
def test_rotated_pack_from_strided_unaligned_rows(align, vrot):
    """The rotated bulk quantizer reads each row 16 bytes per lane: rows only 4-byte
    aligned, or token/head strides that are not multiples of 8 elements, give the
    oracle's bytes; 150 tokens from slot 70 (a partial first tile, a whole one, a
    partial last one) after a 70-token first call."""
    H, grp, kb, vb, n0, n1 = 2, 4, 192, 3, 70, 150
    say("rot pack from views %s vrot %d" % (align, vrot))
    seqs = _batch(H, grp, kb, vb, [n0 + n1], seed=41)
    K, V, _ = seqs[0]
    ksg = synth.rot_signs(H, seed=41)
    vsg = synth.rot_signs(H, seed=42) if vrot else None
    vsig = None
    if not vrot:
        ev = np.zeros((H, D // 2, 2), np.uint64)
        oracle.block_energy(V.numpy(), kvq.PAIR_HALF, ev)
        _, vsig = oracle.allocate(ev, vb * (D // 2), oracle.UNIFORM)
    cap = 256
    g = kvq.geom(H, kb, vb, cap)
    ogeom = oracle.Geometry(H, kb, vb, cap)
    cache = torch.zeros(kvq.cache_bytes(g), dtype=torch.uint8, device="cuda")
    off = torch.zeros(1, dtype=torch.int64, device="cuda")
    _gpu_pack(g, [(K[:n0], V[:n0], None)], [0], ksg, vsg, vsig, cache, off)
    lead = 2 if align == "4byte" else 8
    width = 134 if align == "4byte" else 140
    kb_ = torch.zeros(n0 + n1, H + 1, width, dtype=torch.float16, device="cuda")
    vb_ = torch.zeros_like(kb_)
    kb_[:, :H, lead:lead + D] = K.cuda()
    vb_[:, :H, lead:lead + D] = V.cuda()
    kv, vv = kb_[:, :H, lead:lead + D], vb_[:, :H, lead:lead + D]
    if align == "4byte":
        assert kv.data_ptr() % 16 != 0 and kv.data_ptr() % 4 == 0
    else:
        assert kv.data_ptr() % 16 == 0 and kv.stride(0) % 8 != 0
    kvq.rot_quantize_pack(g, kv, vv, torch.tensor([n0], dtype=torch.int64, device="cuda"),
                          torch.tensor([n1], dtype=torch.int32, device="cuda"),
                          torch.tensor([n0], dtype=torch.int64, device="cuda"), n1, ksg.cuda(),
                          None if vsg is None else vsg.cuda(), None if vsig is None else torch.from_numpy(vsig).cuda(),
                          cache, off)
    oc = np.zeros(ogeom.seq_bytes, np.uint8)
    oracle.quantize_pack_rot(ogeom, oc, K.numpy(), V.numpy(), 0, ksg.numpy(), None if vsg is None else vsg.numpy(),
                             vsig)
    _check_bytes(cache, oc, "views")


def test_rot_abi_rejections():
    g = kvq.geom(2, 160, 3, 128)  # 160 is not a multiple of 64
    q = torch.zeros(1, 4, D, dtype=torch.float16, device="cuda")
    with pytest.raises(kvq.KvqError):
        kvq.rot_queries(g, q, torch.empty_like(q), torch.zeros(2, D, dtype=torch.uint8, device="cuda"))
    g = kvq.geom(2, 192, 16, 128)  # 16-bit values are not rotated
    with pytest.raises(kvq.KvqError):
        kvq.rot_back(g, torch.zeros(1, 4, D, device="cuda"), torch.zeros(2, D, dtype=torch.uint8, device="cuda"))
