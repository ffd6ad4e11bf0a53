"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Energies, widths, scales and packed bytes must match bit for bit; decode
attention must agree per (sequence, query head) within 2e-3 of max|o_ref|.
Shapes span several tiles, ragged tails, empty and one-token sequences, all
budget kinds (K3V3, K2V2, K3V2, K-only V16, K16V16 passthrough, odd budgets),
both RoPE pairings, batches and appends.
"""
import numpy as np
import pytest
import torch

import oracle
from packed_cache_attention_amd import kvq, synth

from pipeline import check_attention, energy_u64, gpu_energy, run_batch, say

pytestmark = pytest.mark.gpu

rng = np.random.default_rng(2024)


def _rand(n, H, d=128, scale=1.0, seed=0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(n, H, d, generator=g, dtype=torch.float64) * scale).to(torch.float16)


def _heads(wl, n, seed=0, seq=0, layer=0):
    return synth.gen_layer(wl, seq, layer, n_tok=n, seed=seed)


# ----------------------------------------------------------------- energy + allocation

@pytest.mark.parametrize("d", [2, 4, 6, 8, 16, 64, 128])
@pytest.mark.parametrize("pairing", [0, 1])
def test_energy_and_allocation_bit_exact(d, pairing):
    say("energy/alloc d=%d pairing=%d" % (d, pairing))
    H = 3
    x = _rand(257, H, d, scale=20.0, seed=d)
    flat = x.view(-1)
    # special values: subnormals, zeros, extremes
    idx = torch.from_numpy(rng.choice(flat.numel(), 12, replace=False))
    flat[idx] = torch.tensor([6e-8, -6e-8, 0.0, -0.0, 65504, -65504, 1e-5, -3e-6, 2.0, -1.0, 1e-7, 300],
                             dtype=torch.float16)
    nb = d // 2
    g = kvq.geom(H, nb * 3 if nb * 3 <= 8 * nb else 0, 3, 0, head_dim=d, rope_pairing=pairing)
    e = gpu_energy(g, [x[:100], x[100:]])
    oe = oracle.block_energy(x.numpy(), pairing)
    np.testing.assert_array_equal(energy_u64(e), oe)
    budgets = sorted(set([0, 1, nb, 3 * nb, 8 * nb, 16 * nb] + list(rng.integers(0, 8 * nb + 1, 6))))
    for budget in budgets:
        for mode in (kvq.GREEDY, kvq.UNIFORM):
            if mode == kvq.UNIFORM and budget % nb and budget != 16 * nb:
                continue
            bits = torch.empty(H, nb, dtype=torch.uint8, device="cuda")
            sig = torch.empty(H, nb, dtype=torch.float32, device="cuda")
            kvq.allocate_bits(g, e, int(budget), mode, bits, sig)
            ob, os_ = oracle.allocate(oe, int(budget), mode)
            np.testing.assert_array_equal(bits.cpu().numpy(), ob, err_msg="budget %d mode %d" % (budget, mode))
            np.testing.assert_array_equal(sig.cpu().numpy().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("d", [16, 128])
def test_allocation_ties_and_zero_energies(d):
    """Energies with many exact ties (equal blocks, blocks whose gains collide across
    widths at powers of two), zero-energy blocks and 128-bit values: widths and
    scales equal the oracle's greedy at every budget."""
    say("alloc ties d=%d" % d)
    nb, H = d // 2, 6
    r = np.random.default_rng(7 + d)
    e = np.zeros((H, nb, 2), np.uint64)
    base = r.integers(1, 1 << 40, size=4, dtype=np.uint64)
    for h in range(H):
        pick = r.integers(0, 4, size=nb)
        e[h, :, 0] = base[pick]                     # only 4 distinct values: ties everywhere
        e[h, r.random(nb) < 0.25, 0] = 0            # zero-energy blocks
        if h % 2:
            e[h, ::3, 0] <<= np.uint64(r.integers(0, 20))  # equal up to a power of two
        if h == 5:
            e[h, :, 1] = r.integers(0, 4, size=nb, dtype=np.uint64)  # values above 2^64
    if H > 0:
        e[0] = 0                                    # an all-zero unit
    g = kvq.geom(H, 0, 3, 0, head_dim=d)
    ed = torch.from_numpy(e.view(np.int64)).cuda()
    for budget in sorted(set([0, 1, 2, nb - 1, nb, nb + 1, 3 * nb, 5 * nb + 3, 8 * nb - 1, 8 * nb])):
        bits = torch.empty(H, nb, dtype=torch.uint8, device="cuda")
        sig = torch.empty(H, nb, dtype=torch.float32, device="cuda")
        kvq.allocate_bits(g, ed, int(budget), kvq.GREEDY, bits, sig)
        ob, os_ = oracle.allocate(e, int(budget), oracle.GREEDY)
        np.testing.assert_array_equal(bits.cpu().numpy(), ob, err_msg="budget %d" % budget)
        np.testing.assert_array_equal(sig.cpu().numpy().view(np.uint32), os_.view(np.uint32))


def test_energy_accumulates_exactly_with_strides():
    say("energy strided")
    H, d = 4, 128
    big = _rand(300, H + 2, d + 8, seed=5)  # padded rows and heads: strides != dense
    x = big[:, 1:H + 1, :d]
    g = kvq.geom(H, 192, 3, 0)
    e = torch.zeros(H, 64, 2, dtype=torch.int64, device="cuda")
    xd = big.cuda()[:, 1:H + 1, :d]
    kvq.block_energy(g, xd, e)
    kvq.block_energy(g, xd, e)  # accumulate twice
    oe = oracle.block_energy(np.ascontiguousarray(x.numpy()))
    oracle.block_energy(np.ascontiguousarray(x.numpy()), energy=oe)
    np.testing.assert_array_equal(energy_u64(e), oe)


# ----------------------------------------------------------------- full pipeline

CASES = [
    # name, H_kv, group, n tokens, capacity, k_budget, v_bits, pairing
    ("k3v3-1tile", 1, 1, 64, 64, 192, 3, 0),
    ("k3v3-ragged", 2, 8, 150, 192, 192, 3, 0),
    ("k2v2-ragged", 2, 4, 321, 384, 128, 2, 0),
    ("k3v2-gqa7", 2, 7, 200, 256, 192, 2, 0),
    ("kodd-v5", 1, 3, 77, 128, 131, 5, 0),
    ("k8v8-max", 1, 2, 130, 192, 512, 8, 0),
    ("k0v1", 1, 2, 65, 128, 0, 1, 0),
    ("konly-v16", 2, 2, 100, 128, 192, 16, 0),
    ("konly-v16-gqa8", 2, 8, 333, 384, 192, 16, 0),
    ("konly-v16-k4-il", 1, 6, 200, 256, 256, 16, 1),
    ("k16v16-pass", 1, 4, 90, 128, 1024, 16, 0),
    ("interleaved", 2, 2, 140, 192, 160, 4, 1),
    ("gqa16", 1, 16, 70, 128, 192, 3, 0),
]


@pytest.mark.parametrize("kernel", [kvq.DECODE_AUTO, kvq.DECODE_GENERIC], ids=["auto", "generic"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pipeline_matches_oracle(case, kernel):
    name, H, grp, n, cap, kb, vb, pairing = case
    say("pipeline %s kernel=%d" % (name, kernel))
    wl = synth.Workload(name, 1, H * grp, H, 1e6, (n,), kb, vb, "decay")
    K, V, q = _heads(wl, n, seed=7)
    if pairing == 1:  # the generator rotates half-split planes; any fp16 keys are valid input
        K = K[:, :, torch.randperm(128, generator=torch.Generator().manual_seed(3))].contiguous()
    run_batch([(K, V, q)], kb, vb, cap, pairing=pairing, kernel=kernel)


def test_passthrough_attention_is_exact_softmax():
    """K16V16: decode attention equals fp64 softmax attention of the fp16 cache."""
    say("passthrough exact")
    H, grp, n = 2, 3, 150
    K, V = _rand(n, H, seed=11), _rand(n, H, seed=12)
    q = _rand(H * grp, 1, seed=13)[:, 0, :]
    r = run_batch([(K, V, q)], 1024, 16, 192, oracle_attn=False)
    for h in range(H * grp):
        k = K[:, h // grp].double().numpy()
        v = V[:, h // grp].double().numpy()
        z = k @ q[h].double().numpy() / np.sqrt(128)
        p = np.exp(z - z.max())
        ref = (p / p.sum()) @ v
        check_attention(r["out"][0, h][None], ref[None])


def test_c1_configuration():
    wl = synth.WORKLOADS["c1"]
    say("c1 %s" % wl.name)
    K, V, q = synth.gen_layer(wl, 0, 0)
    run_batch([(K, V, q)], wl.k_budget, wl.v_bits, 1024)


def test_batch_ragged_lengths():
    """A batch of sequences of different lengths (one allocation shared per head)."""
    say("batch ragged")
    wl = synth.Workload("batch", 1, 14, 2, 1e6, (0,), 192, 2, "decay")
    lens = [1, 63, 64, 65, 200, 0, 129]
    seqs = []
    for s, n in enumerate(lens):
        K, V, q = synth.gen_layer(wl.with_lens(lens), s, 0, n_tok=n, seed=3)
        seqs.append((K, V, q))
    r = run_batch(seqs, 192, 2, 256)
    assert np.all(r["out"][5] == 0)  # empty sequence -> zeros


def test_appends_equal_bulk_and_decode_after_append():
    """Bulk quantization, then token-by-token and chunked appends at ragged slots,
    give the same bytes as the oracle's bulk quantization of all tokens."""
    say("appends")
    wl = synth.Workload("app", 1, 8, 2, 1e6, (0,), 192, 3, "decay")
    n0, n1 = 70, 60
    K, V, q = synth.gen_layer(wl.with_lens([n0 + n1]), 0, 0, n_tok=n0 + n1, seed=9)
    r = run_batch([(K[:n0], V[:n0], q)], 192, 3, 256, check_attn=False)
    g, cache, off = r["g"], r["cache"], r["off"]
    Kd, Vd = K.cuda(), V.cuda()
    slot = n0
    chunks = [1, 1, 5, 17, 1, 35]
    for c in chunks:
        first = torch.tensor([slot], dtype=torch.int64, device="cuda")
        nn = torch.tensor([c], dtype=torch.int32, device="cuda")
        src = torch.tensor([slot], dtype=torch.int64, device="cuda")
        kvq.quantize_pack(g, Kd, Vd, first, nn, src, c, r["kbits"], r["ksig"], r["vsig"], cache, off)
        slot += c
    assert slot == n0 + n1
    oc = np.zeros_like(r["oc"])
    oracle.quantize_pack(r["ogeom"], oc, K.numpy(), V.numpy(), 0, r["ob"], r["osig"], r["ovsig"])
    np.testing.assert_array_equal(cache.cpu().numpy(), oc)
    # invalid device-side entries are skipped (slot beyond capacity)
    first = torch.tensor([250], dtype=torch.int64, device="cuda")
    nn = torch.tensor([10], dtype=torch.int32, device="cuda")
    kvq.quantize_pack(g, Kd, Vd, first, nn, first, 10, r["kbits"], r["ksig"], r["vsig"], cache, off)
    np.testing.assert_array_equal(cache.cpu().numpy(), oc)
    # decode over the appended cache
    seq_len = torch.tensor([n0 + n1], dtype=torch.int32, device="cuda")
    ws = torch.empty(kvq.decode_workspace_bytes(g, 8, 1, 256) // 4, dtype=torch.float32, device="cuda")
    out = torch.empty(1, 8, 128, dtype=torch.float32, device="cuda")
    kvq.packed_decode_attn(g, q[None].cuda().contiguous(), cache, off, seq_len, 256, r["kbits"], r["ksig"],
                           r["vsig"], out, ws)
    ref = oracle.decode_attention(r["ogeom"], oc, q.numpy(), n0 + n1, r["ob"], r["osig"], r["ovsig"])
    check_attention(out.cpu().numpy()[0], ref)


APPEND_CASES = [(c[0], c[5], c[6], c[7]) for c in CASES if c[0] in
                ("k3v3-ragged", "k2v2-ragged", "kodd-v5", "k8v8-max", "k0v1", "konly-v16", "k16v16-pass",
                 "interleaved")]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_small_appends_match_bulk(case):
    """Appends of 1..4 tokens (the one-wave append path) into two sequences at ragged
    slots, across tile boundaries, give the oracle's bulk bytes."""
    name, kb, vb, pairing = case
    say("small appends %s" % name)
    H, n0, n1 = 2, (61, 3), (9, 70)
    wl = synth.Workload("app-" + name, 1, 4, H, 1e6, (0,), kb, vb, "decay")
    seqs = []
    for i in range(2):
        K, V, q = synth.gen_layer(wl.with_lens([n0[i] + n1[i]]), i, 0, n_tok=n0[i] + n1[i], seed=11 + i)
        if pairing == 1:
            K = K[:, :, torch.randperm(128, generator=torch.Generator().manual_seed(5))].contiguous()
        seqs.append((K, V, q))
    # bulk-quantize the first n0 tokens of each sequence (allocation from those tokens)
    r = run_batch([(K[:n0[i]], V[:n0[i]], q) for i, (K, V, q) in enumerate(seqs)], kb, vb, 128, pairing=pairing,
                  check_attn=False)
    g, cache, off = r["g"], r["cache"], r["off"]
    rows = torch.cat([K for K, _, _ in seqs], 0).cuda()
    vrows = torch.cat([V for _, V, _ in seqs], 0).cuda()
    base = [0, n0[0] + n1[0]]
    done = list(n0)
    step = 0
    while done[0] < n0[0] + n1[0] or done[1] < n0[1] + n1[1]:
        c = [min(1 + (step + i) % 4, n0[i] + n1[i] - done[i]) for i in range(2)]
        first = torch.tensor(done, dtype=torch.int64, device="cuda")
        nn = torch.tensor(c, dtype=torch.int32, device="cuda")
        src = torch.tensor([base[i] + done[i] for i in range(2)], dtype=torch.int64, device="cuda")
        kvq.quantize_pack(g, rows, vrows, first, nn, src, 4, r["kbits"], r["ksig"], r["vsig"], cache, off)
        done = [done[i] + c[i] for i in range(2)]
        step += 1
    region = kvq.cache_bytes(g)
    oc = np.zeros(2 * region, np.uint8)
    for i, (K, V, _) in enumerate(seqs):
        oracle.quantize_pack(r["ogeom"], oc[i * region:(i + 1) * region], K.numpy(), V.numpy(), 0, r["ob"], r["osig"],
                             r["ovsig"])
    np.testing.assert_array_equal(cache.cpu().numpy(), oc)


BULK_VIEW_CASES = [(c[0], c[5], c[6], c[7]) for c in CASES if c[0] in
                   ("k3v3-ragged", "k8v8-max", "konly-v16", "k16v16-pass", "interleaved")]


@pytest.mark.parametrize("align", ["4byte", "16byte-oddstride"])
@pytest.mark.parametrize("case", BULK_VIEW_CASES, ids=[c[0] for c in BULK_VIEW_CASES])
def test_bulk_quantize_from_strided_unaligned_rows(case, align):
    """Bulk quantize+pack of 150 tokens starting mid-tile (slot 70: a partial first
    tile, a whole tile, a partial last tile) from K/V views whose rows are only 4-byte
    aligned or whose token/head strides are not multiples of 8 elements gives the
    oracle's bytes for the whole sequence."""
    name, kb, vb, pairing = case
    say("bulk from views %s %s" % (name, align))
    H, n0, n1 = 2, 70, 150
    wl = synth.Workload("views-" + name, 1, 4, H, 1e6, (0,), kb, vb, "decay")
    K, V, q = synth.gen_layer(wl.with_lens([n0 + n1]), 0, 0, n_tok=n0 + n1, seed=21)
    r = run_batch([(K[:n0], V[:n0], q)], kb, vb, 256, pairing=pairing, check_attn=False)
    g, cache, off = r["g"], r["cache"], r["off"]
    lead = 2 if align == "4byte" else 8   # element offset of coordinate 0 within a padded row
    width = 134 if align == "4byte" else 140
    kb_ = torch.zeros(n0 + n1, H + 1, width, dtype=torch.float16, device="cuda")
    vb_ = torch.zeros_like(kb_)
    kb_[:, :H, lead:lead + 128] = K.cuda()
    vb_[:, :H, lead:lead + 128] = V.cuda()
    kv, vv = kb_[:, :H, lead:lead + 128], vb_[:, :H, lead:lead + 128]
    if align == "4byte":
        assert kv.data_ptr() % 16 != 0 and kv.data_ptr() % 4 == 0
    else:
        assert kv.data_ptr() % 16 == 0 and kv.stride(0) % 8 != 0
    assert kv.stride(1) % 8 != 0 or kv.stride(0) % 8 != 0
    first = torch.tensor([n0], dtype=torch.int64, device="cuda")
    nn = torch.tensor([n1], dtype=torch.int32, device="cuda")
    src = torch.tensor([n0], dtype=torch.int64, device="cuda")
    kvq.quantize_pack(g, kv, vv, first, nn, src, n1, r["kbits"], r["ksig"], r["vsig"], cache, off)
    oc = np.zeros_like(r["oc"])
    oracle.quantize_pack(r["ogeom"], oc, K.numpy(), V.numpy(), 0, r["ob"], r["osig"], r["ovsig"])
    np.testing.assert_array_equal(cache.cpu().numpy(), oc)


@pytest.mark.parametrize("kernel", [kvq.DECODE_GENERIC, kvq.DECODE_MFMA])
def test_split_count_invariance(kernel):
    """Any split of the token axis gives the same output up to fp32 re-association (1e-5 of max|o|)."""
    say("split invariance kernel=%d" % kernel)
    wl = synth.Workload("split", 1, 8, 1, 1e6, (0,), 192, 3, "decay")
    n = 1000
    K, V, q = synth.gen_layer(wl.with_lens([n]), 0, 0, n_tok=n, seed=4)
    r = run_batch([(K, V, q)], 192, 3, 1024, kernel=kernel, tiles=1)
    base = r["out"]
    for tiles in (2, 3, 5, 16):
        r2 = run_batch([(K, V, q)], 192, 3, 1024, kernel=kernel, tiles=tiles, oracle_attn=False)
        np.testing.assert_allclose(r2["out"], base, rtol=0, atol=1e-5 * np.abs(base).max())


@pytest.mark.parametrize("kernel", [kvq.DECODE_MFMA, kvq.DECODE_GENERIC])
def test_c2_full_size(kernel):
    """Llama-3.1-8B-shaped layer: 32 q / 8 KV heads, 32K tokens, K2V2 -- every stage."""
    wl = synth.WORKLOADS["c2"]
    say("c2 full %s kernel=%d" % (wl.name, kernel))
    K, V, q = synth.gen_layer(wl, 0, 0)
    run_batch([(K, V, q)], wl.k_budget, wl.v_bits, 32768, kernel=kernel)


# ----------------------------------------------------------------- the model-shaped workloads at full size

@pytest.mark.parametrize("layer", [0, 17, 35])
def test_c3_full_size_sampled_layers(layer):
    """Qwen2.5-3B-shaped 128K K3V3 (the bench workload): one layer per case at its
    full 131072-token context, every stage against the oracle, decode in the
    automatic launch plan the bench uses."""
    wl = synth.WORKLOADS["c3"]
    say("c3 full layer %d" % layer)
    K, V, q = synth.gen_layer(wl, 0, layer)
    n = K.shape[0]
    r = run_batch([(K, V, q)], wl.k_budget, wl.v_bits, synth.ceil_to(n + 64, 64))
    say("c3 layer %d: attention ok, worst rel %.2e" % (layer, check_attention(r["out"], r["ref"])))


@pytest.mark.parametrize("v_bits", [3, 16], ids=["k3v3", "konly-v16"])
def test_c3_full_size_fused_step_as_benchmarked(v_bits):
    """The launch the benchmark times, at its size: one 128K Qwen2.5-3B-shaped layer,
    kvq_decode_step (the new token quantized and packed inside the attention kernel,
    then the split merge) in the automatic plan with max_len = capacity; the cache
    bytes against the oracle's packing of the same token into its own copy, the
    output against its attention over all n + 1 tokens.  Also in the K-only value
    mode (16-bit values), the bench's labelled K-only line."""
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["c3"], v_bits=v_bits)
    layer = 17
    say("c3 full-size fused step, layer %d" % layer)
    K, V, _ = synth.gen_layer(wl, 0, layer)
    n = K.shape[0]
    kn, vn, qn = synth.gen_new_token(wl, 0, layer, n, 0)
    cap = synth.ceil_to(n + 64, 64)
    r = run_batch([(K, V, qn)], wl.k_budget, wl.v_bits, cap, check_attn=False)
    g, region = r["g"], kvq.cache_bytes(r["g"])
    plan = kvq.decode_plan(g, wl.n_q_heads, 1, cap)
    say("plan %s" % plan)
    assert plan["kernel"] == kvq.DECODE_MFMA
    ws = torch.empty(plan["workspace"] // 4 + 4, dtype=torch.float32, device="cuda")
    out = torch.empty(1, wl.n_q_heads, 128, dtype=torch.float32, device="cuda")
    kvq.decode_step(g, qn[None].cuda().contiguous(), kn[None].cuda().contiguous(), vn[None].cuda().contiguous(),
                    r["cache"], r["off"], torch.tensor([n + 1], dtype=torch.int32, device="cuda"), cap, r["kbits"],
                    r["ksig"], r["vsig"], out, ws)
    oc = r["oc"].copy()
    oracle.quantize_pack(r["ogeom"], oc[:region], kn[None].numpy(), vn[None].numpy(), n, r["ob"], r["osig"],
                         r["ovsig"])
    np.testing.assert_array_equal(r["cache"].cpu().numpy(), oc)
    ref = oracle.decode_attention(r["ogeom"], oc[:region], qn.numpy(), n + 1, r["ob"], r["osig"], r["ovsig"])
    say("c3 fused step: bytes ok, attention worst rel %.2e" % check_attention(out.cpu().numpy(), ref[None]))


def test_c4_full_size_layer0():
    """The same shape at 524288 tokens (one layer): long-context tiling and the split merge."""
    wl = synth.WORKLOADS["c4"]
    say("c4 full layer 0")
    K, V, q = synth.gen_layer(wl, 0, 0)
    run_batch([(K, V, q)], wl.k_budget, wl.v_bits, synth.ceil_to(K.shape[0] + 64, 64))


def test_c5_batch_append_then_attend():
    """R1-Distill-Qwen-7B-shaped batch (28 q / 4 KV heads, 16 sequences of 4K..32K,
    K3V2), one layer: bulk prefill, then the decode step's append of one token per
    sequence, then attention over the n+1 tokens -- bytes and outputs against the
    oracle's quantization of all n+1 tokens."""
    wl = synth.WORKLOADS["c5"]
    layer = 27
    say("c5 batch layer %d" % layer)
    seqs, new = [], []
    for s, n in enumerate(wl.seq_lens):
        K, V, q = synth.gen_layer(wl, s, layer)
        kn, vn, qn = synth.gen_new_token(wl, s, layer, n, 0)
        seqs.append((K, V, q))
        new.append((kn, vn, qn))
    cap = synth.ceil_to(max(wl.seq_lens) + 64, 64)
    r = run_batch(seqs, wl.k_budget, wl.v_bits, cap, check_attn=False)
    g, cache, off = r["g"], r["cache"], r["off"]
    S, H, d = len(seqs), wl.n_kv_heads, 128
    kn = torch.stack([x[0] for x in new]).cuda()
    vn = torch.stack([x[1] for x in new]).cuda()
    lens = torch.tensor(wl.seq_lens, dtype=torch.int64, device="cuda")
    kvq.quantize_pack(g, kn, vn, lens, torch.ones(S, dtype=torch.int32, device="cuda"),
                      torch.arange(S, dtype=torch.int64, device="cuda"), 1, r["kbits"], r["ksig"], r["vsig"], cache,
                      off)
    region = kvq.cache_bytes(g)
    oc = np.zeros(S * region, np.uint8)
    for i, ((K, V, _), (k1, v1, _)) in enumerate(zip(seqs, new)):
        oracle.quantize_pack(r["ogeom"], oc[i * region:(i + 1) * region], torch.cat([K, k1[None]]).numpy(),
                             torch.cat([V, v1[None]]).numpy(), 0, r["ob"], r["osig"], r["ovsig"])
    np.testing.assert_array_equal(cache.cpu().numpy(), oc)
    say("c5: appended bytes ok")
    q = torch.stack([x[2] for x in new]).cuda().contiguous()
    seq_len = (lens + 1).to(torch.int32)
    ws = torch.empty(kvq.decode_workspace_bytes(g, wl.n_q_heads, S, cap) // 4, dtype=torch.float32, device="cuda")
    out = torch.empty(S, wl.n_q_heads, d, dtype=torch.float32, device="cuda")
    kvq.packed_decode_attn(g, q, cache, off, seq_len, cap, r["kbits"], r["ksig"], r["vsig"], out, ws)
    ref = np.stack([oracle.decode_attention(r["ogeom"], oc[i * region:(i + 1) * region], new[i][2].numpy(),
                                            wl.seq_lens[i] + 1, r["ob"], r["osig"], r["ovsig"]) for i in range(S)])
    say("c5: attention worst rel %.2e" % check_attention(out.cpu().numpy(), ref))


STEP_CASES = [(c[0], c[1], c[2], c[5], c[6], c[7]) for c in CASES if c[0] in
              ("k3v3-ragged", "k2v2-ragged", "kodd-v5", "k8v8-max", "k0v1", "konly-v16", "konly-v16-gqa8",
               "konly-v16-k4-il", "k16v16-pass", "interleaved", "gqa16")]


@pytest.mark.parametrize("tiles", [0, 1, 4, 8])
@pytest.mark.parametrize("case", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_decode_step_equals_append_then_attend(case, tiles):
    """kvq_decode_step (append inside the attention kernel where it applies) gives the
    bytes and outputs of kvq_quantize_pack followed by kvq_packed_decode_attn, over
    three steps whose new tokens cross tile boundaries (appending waves 0-3, and a wave
    whose tail tile is its second), and the oracle's attention."""
    name, H, grp, kb, vb, pairing = case
    say("decode step %s tiles=%d" % (name, tiles))
    n0 = [62, 127, 1, 200, 290]
    steps = 3
    wl = synth.Workload("step-" + name, 1, H * grp, H, 1e6, (0,), kb, vb, "decay")
    seqs = []
    for i, n in enumerate(n0):
        K, V, q = synth.gen_layer(wl.with_lens([n + steps]), i, 0, n_tok=n + steps, seed=21 + i)
        if pairing == 1:
            K = K[:, :, torch.randperm(128, generator=torch.Generator().manual_seed(8))].contiguous()
        seqs.append((K, V, q))
    cap = 384
    r = run_batch([(K[:n], V[:n], q) for (K, V, q), n in zip(seqs, n0)], kb, vb, cap, pairing=pairing,
                  check_attn=False)
    g, off = r["g"], r["off"]
    S = len(seqs)
    cache_a, cache_b = r["cache"].clone(), r["cache"].clone()
    nq = H * grp
    ws = torch.empty(kvq.decode_workspace_bytes(g, nq, S, cap, kvq.DECODE_AUTO, tiles) // 4, dtype=torch.float32,
                     device="cuda")
    region = kvq.cache_bytes(g)
    for st in range(steps):
        kn = torch.stack([K[n0[i] + st] for i, (K, _, _) in enumerate(seqs)]).cuda()
        vn = torch.stack([V[n0[i] + st] for i, (_, V, _) in enumerate(seqs)]).cuda()
        q = torch.stack([x[2] for x in seqs]).cuda().contiguous()
        lens = torch.tensor([n + st for n in n0], dtype=torch.int64, device="cuda")
        seq_len = (lens + 1).to(torch.int32)
        # the two calls
        kvq.quantize_pack(g, kn, vn, lens, torch.ones(S, dtype=torch.int32, device="cuda"),
                          torch.arange(S, dtype=torch.int64, device="cuda"), 1, r["kbits"], r["ksig"], r["vsig"],
                          cache_a, off)
        out_a = torch.empty(S, nq, 128, dtype=torch.float32, device="cuda")
        kvq.packed_decode_attn(g, q, cache_a, off, seq_len, cap, r["kbits"], r["ksig"], r["vsig"], out_a, ws,
                               tiles_per_split=tiles)
        # the fused step
        out_b = torch.empty_like(out_a)
        kvq.decode_step(g, q, kn, vn, cache_b, off, seq_len, cap, r["kbits"], r["ksig"], r["vsig"], out_b, ws,
                        tiles_per_split=tiles)
        np.testing.assert_array_equal(cache_b.cpu().numpy(), cache_a.cpu().numpy())
        np.testing.assert_array_equal(out_b.cpu().numpy(), out_a.cpu().numpy())
    # and both equal the oracle's quantization of every token, and its attention
    oc = np.zeros(S * region, np.uint8)
    for i, (K, V, _) in enumerate(seqs):
        oracle.quantize_pack(r["ogeom"], oc[i * region:(i + 1) * region], K.numpy(), V.numpy(), 0, r["ob"], r["osig"],
                             r["ovsig"])
    np.testing.assert_array_equal(cache_b.cpu().numpy(), oc)
    ref = np.stack([oracle.decode_attention(r["ogeom"], oc[i * region:(i + 1) * region], seqs[i][2].numpy(),
                                            n0[i] + steps, r["ob"], r["osig"], r["ovsig"]) for i in range(S)])
    check_attention(out_b.cpu().numpy(), ref)


def test_layer_batched_geometry_equals_per_layer_calls():
    """The bench's layer-batched capability reading: L layers' regions laid end to end
    are one region of L * H_kv KV heads, so one decode call over that geometry gives
    each layer's per-layer result (up to the merge order)."""
    L, H, grp, kb, vb, n = 3, 2, 8, 192, 3, 700
    wl = synth.Workload("lb", L, H * grp, H, 1e6, (n,), kb, vb, "decay")
    cap = synth.ceil_to(n + 64, 64)
    per_layer, caches, bits, ks, vs, qs = [], [], [], [], [], []
    for l in range(L):
        K, V, q = synth.gen_layer(wl, 0, l)
        r = run_batch([(K, V, q)], kb, vb, cap)
        per_layer.append(r["out"][0])
        caches.append(r["cache"]); bits.append(r["kbits"]); ks.append(r["ksig"]); vs.append(r["vsig"])
        qs.append(q)
    gb = kvq.geom(L * H, kb, vb, cap)
    cache = torch.cat(caches).contiguous()
    q = torch.cat(qs)[None].cuda().contiguous()
    out = torch.empty(1, L * H * grp, 128, dtype=torch.float32, device="cuda")
    ws = torch.empty(kvq.decode_workspace_bytes(gb, L * H * grp, 1, n) // 4 + 4, dtype=torch.float32, device="cuda")
    kvq.packed_decode_attn(gb, q, cache, torch.zeros(1, dtype=torch.int64, device="cuda"),
                           torch.tensor([n], dtype=torch.int32, device="cuda"), n, torch.cat(bits), torch.cat(ks),
                           torch.cat(vs), out, ws)
    o = out.cpu().numpy()[0].reshape(L, H * grp, 128)
    for l in range(L):
        np.testing.assert_allclose(o[l], per_layer[l], rtol=0, atol=2e-6 * np.abs(per_layer[l]).max())


def test_read_probe_reads_every_word():
    """The bandwidth probe folds every 16-byte word it reads: with each word's four
    dwords XOR-ed, the XOR of the workgroups' results equals the whole buffer's."""
    g = torch.Generator().manual_seed(3)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (1 << 20,), dtype=torch.int32, generator=g)
    want = np.bitwise_xor.reduce(buf.numpy().view(np.uint32))
    for nb in (1, 7, 256, 2048):
        sink = torch.zeros(nb, dtype=torch.int32, device="cuda")
        kvq.read_probe(buf.cuda(), sink, nb)
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, (nb, got, want)
