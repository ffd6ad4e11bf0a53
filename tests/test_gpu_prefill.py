"""GPU parity for chunked prefill attention over the packed cache (causal): a chunk
of queries at positions q_start .. q_start + n - 1 attends every slot up to its own
position, the chunk itself packed first ("RoPE-Aware Bit Allocation for KV-Cache
Quantization", abstract: at 256K and 512K only the packed cache fits; a prompt of that
length is read here as filled chunk by chunk).  Checked against the oracle's causal attention row by row (2e-3 of the
row's largest output per (sequence, query, head)); rows past a sequence's queries
must be exactly zero.  Cases: GQA groups 1..8 (including 3 and 7, whose 256-row
blocks are not full), K budgets 64..512 (block widths up to 8) and the K16 / V16
passthrough widths (the K-only mode), value widths 1..8,
both RoPE pairings, ragged batches with empty and one-query chunks, chunks at the
start of the context and deep into it, forced key-range splits, and the 128K
Qwen2.5-3B-shaped layer at full size on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
from packed_cache_attention_amd import kvq, synth

from pipeline import check_attention, run_batch, say

pytestmark = pytest.mark.gpu

CASES = [
    # name, H_kv, group, k_budget, v_bits, pairing, [(q_start, n_q)], n_split
    ("k3v3-g8", 2, 8, 192, 3, 0, [(1000, 77)], 0),
    ("k3v3-g8-split3", 2, 8, 192, 3, 0, [(1000, 77)], 3),
    ("k3v3-g8-split1", 2, 8, 192, 3, 0, [(1000, 77)], 1),
    ("k2v2-g4-ragged", 2, 4, 128, 2, 0, [(300, 150), (0, 64)], 0),
    ("k3v2-g7-batch", 2, 7, 192, 2, 0, [(500, 37), (64, 1), (200, 0)], 2),
    ("k4v4-g2-interleaved", 1, 2, 256, 4, 1, [(250, 130)], 0),
    ("k8v8-g1", 1, 1, 512, 8, 0, [(100, 140)], 0),
    ("kodd-v5-g3", 1, 3, 131, 5, 0, [(190, 100)], 0),
    ("k1v1-g8-start", 2, 8, 64, 1, 0, [(0, 200)], 0),
    ("konly-k3-v16-g4", 2, 4, 192, 16, 0, [(260, 70)], 0),
    ("k16v16-g2-passthrough", 1, 2, 1024, 16, 0, [(90, 50), (0, 7)], 2),
]


def _run(H, grp, kb, vb, pairing, chunks, n_split, seed=7, layer=0):
    nq = H * grp
    S = len(chunks)
    wl = synth.Workload("pf", 1, nq, H, 1e6, (0,), kb, vb, "decay")
    lens = [a + n for a, n in chunks]
    seqs = [synth.gen_layer(wl.with_lens([lens[i]]), i, layer, n_tok=lens[i], seed=seed + i) for i in range(S)]
    cap = 64 * ((max(lens) + 63) // 64 + 1)
    # the whole context, chunk included, packed first (bytes checked against the oracle)
    r = run_batch(seqs, kb, vb, cap, pairing=pairing, check_attn=False)
    g, ogeom, region = r["g"], r["ogeom"], kvq.cache_bytes(r["g"])
    max_q = max(n for _, n in chunks)
    q = torch.zeros(S, max(max_q, 1), nq, 128, dtype=torch.float16)
    for i, (a, n) in enumerate(chunks):
        if n:
            q[i, :n] = synth.gen_chunk_queries(wl, i, layer, a, n, seed=seed)
    qd = q.cuda().contiguous()
    out = torch.full(qd.shape, float("nan"), dtype=torch.float32, device="cuda")
    ws_bytes = kvq.prefill_workspace_bytes(g, nq, S, qd.shape[1], max(lens), n_split)
    ws = torch.empty(max(ws_bytes // 4, 4), dtype=torch.float32, device="cuda")
    qs = torch.tensor([a for a, _ in chunks], dtype=torch.int32, device="cuda")
    ns = torch.tensor([n for _, n in chunks], dtype=torch.int32, device="cuda")
    kvq.packed_prefill_attn(g, qd, r["cache"], r["off"], qs, ns, max(lens), r["kbits"], r["ksig"], r["vsig"], out,
                            ws, n_split=n_split)
    o = out.cpu().numpy()
    worst = 0.0
    for i, (a, n) in enumerate(chunks):
        assert (o[i, n:] == 0).all(), "rows past the chunk's queries must be zero"
        if n == 0:
            continue
        ref = oracle.prefill_attention(ogeom, r["oc"][i * region:(i + 1) * region], q[i, :n].numpy(), a,
                                       r["ob"], r["osig"], r["ovsig"])
        worst = max(worst, check_attention(o[i, :n], ref))
    return worst


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(case):
    name, H, grp, kb, vb, pairing, chunks, n_split = case
    say("prefill %s" % name)
    worst = _run(H, grp, kb, vb, pairing, chunks, n_split)
    say("prefill %s ok, worst rel %.2e" % (name, worst))


@pytest.mark.parametrize("nt", [512, 2048])
def test_prefill_c3_full_size_sampled_rows(nt):
    """Qwen2.5-3B-shaped 128K K3V3 layer: the last nt-token chunk of a chunked prefill
    (queries at 131072 - nt .. 131071 over the whole packed context) in the automatic
    plan -- 2048 is the chunk the benchmark times; sampled query rows against the
    oracle's decode attention at each row's length."""
    wl = synth.WORKLOADS["c3"]
    say("prefill c3 full size, chunk %d" % nt)
    K, V, _ = synth.gen_layer(wl, 0, 0)
    n = K.shape[0]
    r = run_batch([(K, V, torch.zeros(wl.n_q_heads, 128, dtype=torch.float16))], wl.k_budget, wl.v_bits,
                  synth.ceil_to(n + 64, 64), check_attn=False)
    g, region = r["g"], kvq.cache_bytes(r["g"])
    a = n - nt
    q = synth.gen_chunk_queries(wl, 0, 0, a, nt).unsqueeze(0).contiguous()
    qd = q.cuda()
    out = torch.empty(qd.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(kvq.prefill_workspace_bytes(g, wl.n_q_heads, 1, nt, n) // 4, 4), dtype=torch.float32,
                     device="cuda")
    kvq.packed_prefill_attn(g, qd, r["cache"], r["off"], torch.tensor([a], dtype=torch.int32, device="cuda"),
                            torch.tensor([nt], dtype=torch.int32, device="cuda"), n, r["kbits"], r["ksig"], r["vsig"],
                            out, ws)
    o = out.cpu().numpy()[0]
    for j in (0, 1, nt // 2 - 1, nt - 1):
        ref = oracle.decode_attention(r["ogeom"], r["oc"][:region], q[0, j].numpy(), a + j + 1, r["ob"], r["osig"],
                                      r["ovsig"])
        say("row %d worst rel %.2e" % (j, check_attention(o[j][None], ref[None])))


def test_prefill_rows_equal_gpu_decode():
    """Both HIP paths on the same packed cache: prefill row j equals the decode kernel's
    output for that query at length q_start + j + 1 (within the attention tolerance)."""
    H, grp, kb, vb = 2, 8, 192, 3
    nq_heads = H * grp
    wl = synth.Workload("pf-dec", 1, nq_heads, H, 1e6, (0,), kb, vb, "decay")
    a, n = 900, 70
    K, V, _ = synth.gen_layer(wl.with_lens([a + n]), 0, 0, n_tok=a + n, seed=3)
    cap = 64 * ((a + n + 63) // 64 + 1)
    r = run_batch([(K, V, torch.zeros(nq_heads, 128, dtype=torch.float16))], kb, vb, cap, check_attn=False)
    g = r["g"]
    q = synth.gen_chunk_queries(wl, 0, 0, a, n, seed=3).unsqueeze(0).contiguous().cuda()
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(kvq.prefill_workspace_bytes(g, nq_heads, 1, n, a + n) // 4, 4), dtype=torch.float32,
                     device="cuda")
    kvq.packed_prefill_attn(g, q, r["cache"], r["off"], torch.tensor([a], dtype=torch.int32, device="cuda"),
                            torch.tensor([n], dtype=torch.int32, device="cuda"), a + n, r["kbits"], r["ksig"],
                            r["vsig"], out, ws)
    rows = [0, 1, 33, 69]
    # the decode kernel: one sequence per sampled row, all sharing the same region
    qd = torch.stack([q[0, j] for j in rows]).contiguous()
    lens = torch.tensor([a + j + 1 for j in rows], dtype=torch.int32, device="cuda")
    off = r["off"][:1].repeat(len(rows)).contiguous()
    dout = torch.empty(len(rows), nq_heads, 128, dtype=torch.float32, device="cuda")
    dws = torch.empty(kvq.decode_workspace_bytes(g, nq_heads, len(rows), a + n) // 4 + 4, dtype=torch.float32,
                      device="cuda")
    kvq.packed_decode_attn(g, qd, r["cache"], off, lens, a + n, r["kbits"], r["ksig"], r["vsig"], dout, dws)
    po = out.cpu().numpy()[0][rows]
    say("prefill vs decode kernel, worst rel %.2e" % check_attention(po, dout.cpu().numpy().astype(np.float64)))


def test_prefill_clamps_query_counts_to_max_q():
    """A sequence whose device query count exceeds max_q is clamped to max_q (no row past
    the output is touched): the result equals the call with n_q = max_q."""
    H, grp, kb, vb = 1, 4, 128, 2
    nq_heads = H * grp
    wl = synth.Workload("pf-clamp", 1, nq_heads, H, 1e6, (0,), kb, vb, "decay")
    a, n = 200, 40
    K, V, _ = synth.gen_layer(wl.with_lens([a + n + 30]), 0, 0, n_tok=a + n + 30, seed=5)
    cap = 64 * ((a + n + 30 + 63) // 64 + 1)
    r = run_batch([(K, V, torch.zeros(nq_heads, 128, dtype=torch.float16))], kb, vb, cap, check_attn=False)
    g = r["g"]
    q = synth.gen_chunk_queries(wl, 0, 0, a, n, seed=5).unsqueeze(0).contiguous().cuda()
    outs = []
    for nqv in (n, n + 30):
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        kvq.packed_prefill_attn(g, q, r["cache"], r["off"], torch.tensor([a], dtype=torch.int32, device="cuda"),
                                torch.tensor([nqv], dtype=torch.int32, device="cuda"), a + n + 30, r["kbits"],
                                r["ksig"], r["vsig"], out, None, n_split=1)
        outs.append(out.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])


def test_prefill_c4_full_size_sampled_rows():
    """The same shape at 524288 tokens: the last 256-query chunk over the whole packed
    context (8193 tiles per KV head, split over workgroups and merged), sampled rows
    against the oracle's decode attention at each row's length."""
    wl = synth.WORKLOADS["c4"]
    say("prefill c4 full size")
    K, V, _ = synth.gen_layer(wl, 0, 0)
    n = K.shape[0]
    r = run_batch([(K, V, torch.zeros(wl.n_q_heads, 128, dtype=torch.float16))], wl.k_budget, wl.v_bits,
                  synth.ceil_to(n + 64, 64), check_attn=False)
    g, region = r["g"], kvq.cache_bytes(r["g"])
    nt = 256
    a = n - nt
    q = synth.gen_chunk_queries(wl, 0, 0, a, nt).unsqueeze(0).contiguous()
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    plan = kvq.prefill_plan(g, wl.n_q_heads, 1, nt, n)
    say("plan %s" % plan)
    ws = torch.empty(max(plan["workspace"] // 4, 4), dtype=torch.float32, device="cuda")
    kvq.packed_prefill_attn(g, q.cuda(), r["cache"], r["off"], torch.tensor([a], dtype=torch.int32, device="cuda"),
                            torch.tensor([nt], dtype=torch.int32, device="cuda"), n, r["kbits"], r["ksig"], r["vsig"],
                            out, ws)
    o = out.cpu().numpy()[0]
    for j in (0, 255):
        ref = oracle.decode_attention(r["ogeom"], r["oc"][:region], q[0, j].numpy(), a + j + 1, r["ob"], r["osig"],
                                      r["ovsig"])
        say("row %d worst rel %.2e" % (j, check_attention(o[j][None], ref[None])))
