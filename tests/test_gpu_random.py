"""Seeded random sweep over valid geometries, through the C ABI, against the oracle.

Each seed draws a geometry -- KV heads 1..4, GQA group 1..8, 12 or 16, K budget 0..512
or the K16 passthrough, value width 1..8 or 16, either RoPE pairing -- and a ragged
batch of 1..4 sequences of 0..500 tokens (empty ones included).  Checked: energies,
widths, scales and packed bytes bit for bit, decode attention in the automatic plan
and at a random chunk size, and chunked-prefill attention of each sequence's tail
from a random start, all within 2e-3 of the oracle's per-head output (the parity bar of "RoPE-Aware Bit Allocation for KV-Cache
Quantization"'s packed serving path as read here)."""
import numpy as np
import pytest
import torch

import oracle
from packed_cache_attention_amd import kvq, synth

from pipeline import check_attention, run_batch, say

pytestmark = pytest.mark.gpu

SEEDS = list(range(14))


def _draw(seed):
    r = np.random.default_rng(1000 + seed)
    H = int(r.integers(1, 5))
    grp = int(r.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
    kb = 1024 if r.random() < 0.1 else int(r.integers(0, 513))
    vb = 16 if r.random() < 0.15 else int(r.integers(1, 9))
    pairing = int(r.integers(0, 2))
    S = int(r.integers(1, 5))
    lens = [int(x) for x in r.integers(0, 501, S)]
    if max(lens) == 0:
        lens[0] = int(r.integers(1, 200))
    tiles = int(r.choice([0, 4, 8, 12]))
    return H, grp, kb, vb, pairing, lens, tiles, r


@pytest.mark.parametrize("seed", SEEDS)
def test_random_geometry_decode_and_prefill(seed):
    H, grp, kb, vb, pairing, lens, tiles, r = _draw(seed)
    say("random seed %d: H %d group %d K budget %d V %d pairing %d lengths %s tiles %d"
        % (seed, H, grp, kb, vb, pairing, lens, tiles))
    nq = H * grp
    wl = synth.Workload("rand", 1, nq, H, 1e6, (0,), kb, vb, "decay")
    seqs = [synth.gen_layer(wl.with_lens([n]), i, 0, n_tok=n, seed=50 + seed) for i, n in enumerate(lens)]
    cap = 64 * ((max(lens) + 63) // 64 + 1)
    # every stage bit-exact, decode attention in the automatic plan
    res = run_batch(seqs, kb, vb, cap, pairing=pairing)
    g, off, region = res["g"], res["off"], kvq.cache_bytes(res["g"])
    # decode at a chosen chunk size (the kernel the plan picks for it)
    if tiles:
        q = torch.stack([s[2] for s in seqs]).cuda().contiguous()
        seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
        ws = torch.empty(kvq.decode_workspace_bytes(g, nq, len(lens), max(lens), kvq.DECODE_AUTO, tiles) // 4 + 4,
                         dtype=torch.float32, device="cuda")
        out = torch.empty(len(lens), nq, 128, dtype=torch.float32, device="cuda")
        kvq.packed_decode_attn(g, q, res["cache"], off, seq_len, max(lens), res["kbits"], res["ksig"], res["vsig"],
                               out, ws, tiles_per_split=tiles)
        check_attention(out.cpu().numpy(), res["ref"])
    # chunked prefill: each sequence's tail from a random start (empty chunks included)
    starts = [int(r.integers(0, n + 1)) for n in lens]
    nqs = [n - a for n, a in zip(lens, starts)]
    max_q = max(max(nqs), 1)
    qp = torch.zeros(len(lens), max_q, nq, 128, dtype=torch.float16)
    for i, (a, n) in enumerate(zip(starts, nqs)):
        if n:
            qp[i, :n] = synth.gen_chunk_queries(wl, i, 0, a, n, seed=seed)
    n_split = int(r.choice([0, 1, 2, 5]))
    pws = torch.empty(max(kvq.prefill_workspace_bytes(g, nq, len(lens), max_q, max(lens), n_split) // 4, 4),
                      dtype=torch.float32, device="cuda")
    pout = torch.full(qp.shape, float("nan"), dtype=torch.float32, device="cuda")
    kvq.packed_prefill_attn(g, qp.cuda().contiguous(), res["cache"], off,
                            torch.tensor(starts, dtype=torch.int32, device="cuda"),
                            torch.tensor(nqs, dtype=torch.int32, device="cuda"), max(lens), res["kbits"],
                            res["ksig"], res["vsig"], pout, pws, n_split=n_split)
    po = pout.cpu().numpy()
    worst = 0.0
    for i, (a, n) in enumerate(zip(starts, nqs)):
        assert (po[i, n:] == 0).all()
        if n == 0:
            continue
        ref = oracle.prefill_attention(res["ogeom"], res["oc"][i * region:(i + 1) * region], qp[i, :n].numpy(), a,
                                       res["ob"], res["osig"], res["ovsig"])
        worst = max(worst, check_attention(po[i, :n], ref))
    say("random seed %d ok (prefill worst rel %.2e)" % (seed, worst))
