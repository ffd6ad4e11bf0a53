"""GPU parity with value rows of large norm.  The matrix-core kernels feed p * s^V (the
softmax weight times the token's value norm) to the matrix cores as binary16; these
cases put value norms from 10^2 to the largest a binary16 row can have (every
coordinate +-60000: norm 6.8e5) through the automatic decode, the fused decode step
(the appended token among them), the fp16-window step and chunked prefill, against
the oracle's exact attention ("RoPE-Aware Bit Allocation for KV-Cache Quantization",
abstract: the packed-cache serving path reads whatever values the model caches).
Queries are scaled up so logits spread and the lazy running maximum leaves weights
near its 2^8 slack."""
import numpy as np
import pytest
import torch

import oracle
from packed_cache_attention_amd import kvq, synth

from pipeline import check_attention, run_batch, say

pytestmark = pytest.mark.gpu

BIG = 60000.0


def big_values(V: torch.Tensor, seed: int, mode: str) -> torch.Tensor:
    """V [n, H, d] fp16 -> values of large norm: "loguniform" scales every token by
    10^U(2, 3.6); "outliers" keeps N(0, 1) rows but turns a few tokens (one of them the
    last) into +-60000 rows; "both" does both."""
    g = torch.Generator().manual_seed(seed)
    n, H, d = V.shape
    x = V.to(torch.float64)
    if mode in ("loguniform", "both"):
        x = x * (10.0 ** (2.0 + 1.6 * torch.rand(n, H, 1, generator=g, dtype=torch.float64)))
    if mode in ("outliers", "both"):
        idx = torch.cat([torch.randint(0, n, (3,), generator=g), torch.tensor([n - 1])])
        sign = torch.randint(0, 2, (len(idx), H, d), generator=g, dtype=torch.float64) * 2 - 1
        x[idx] = sign * BIG
    return x.clamp(-65504, 65504).to(torch.float16)


def _seqs(lens, H, grp, kb, vb, mode, seed, qscale=3.0):
    wl = synth.Workload("vn", 1, H * grp, H, 1e6, (0,), kb, vb, "decay")
    out = []
    for i, n in enumerate(lens):
        K, V, q = synth.gen_layer(wl.with_lens([n]), i, 0, n_tok=n, seed=seed + i)
        q = (q.to(torch.float32) * qscale).to(torch.float16)
        out.append((K, big_values(V, seed + 100 + i, mode), q))
    return out


@pytest.mark.parametrize("mode", ["loguniform", "outliers", "both"])
@pytest.mark.parametrize("geom", [(2, 8, 192, 3), (2, 4, 128, 2), (1, 7, 131, 5), (2, 8, 192, 16)],
                         ids=["k3v3g8", "k2v2g4", "kodd-v5g7", "konly-v16g8"])
@pytest.mark.parametrize("tiles", [0, 1])
def test_decode_large_value_norms(mode, geom, tiles):
    H, grp, kb, vb = geom
    say("value norms: decode %s %s tiles %d" % (mode, geom, tiles))
    seqs = _seqs((1000, 333, 64), H, grp, kb, vb, mode, seed=11)
    r = run_batch(seqs, kb, vb, 1088, tiles=tiles)
    assert np.isfinite(r["out"]).all()
    say("worst rel %.2e" % check_attention(r["out"], r["ref"]))


@pytest.mark.parametrize("vb", [3, 16], ids=["v3", "v16"])
@pytest.mark.parametrize("mode", ["outliers", "both"])
def test_decode_step_appends_large_norm_token(mode, vb):
    """The fused step packs a new token of the largest value norm inside the attention
    kernel and attends it with the rest (3-bit and 16-bit values)."""
    say("value norms: fused step %s v%d" % (mode, vb))
    H, grp, kb = 2, 8, 192
    lens = (700, 129)
    seqs = _seqs([n + 1 for n in lens], H, grp, kb, vb, mode, seed=23)
    r = run_batch([(K[:n], V[:n], q) for (K, V, q), n in zip(seqs, lens)], kb, vb, 832, check_attn=False)
    g, region = r["g"], kvq.cache_bytes(r["g"])
    kn = torch.stack([K[n] for (K, _, _), n in zip(seqs, lens)]).cuda()
    vn = torch.stack([torch.full_like(V[n], BIG) * torch.sign(V[n].float() + 0.5).half() for (_, V, _), n
                      in zip(seqs, lens)]).cuda()
    q = torch.stack([x[2] for x in seqs]).cuda().contiguous()
    seq_len = torch.tensor([n + 1 for n in lens], dtype=torch.int32, device="cuda")
    ws = torch.empty(kvq.decode_workspace_bytes(g, H * grp, 2, 832) // 4 + 4, dtype=torch.float32, device="cuda")
    out = torch.empty(2, H * grp, 128, dtype=torch.float32, device="cuda")
    kvq.decode_step(g, q, kn, vn, r["cache"], r["off"], seq_len, 832, r["kbits"], r["ksig"], r["vsig"], out, ws)
    oc = r["oc"].copy()
    for i, n in enumerate(lens):
        oracle.quantize_pack(r["ogeom"], oc[i * region:(i + 1) * region], kn[i:i + 1].cpu().numpy(),
                             vn[i:i + 1].cpu().numpy(), n, r["ob"], r["osig"], r["ovsig"])
    np.testing.assert_array_equal(r["cache"].cpu().numpy(), oc)
    ref = np.stack([oracle.decode_attention(r["ogeom"], oc[i * region:(i + 1) * region], seqs[i][2].numpy(),
                                            lens[i] + 1, r["ob"], r["osig"], r["ovsig"]) for i in range(2)])
    o = out.cpu().numpy()
    assert np.isfinite(o).all()
    say("worst rel %.2e" % check_attention(o, ref))


def test_window_step_large_value_norms():
    """fp16 window W = 48: packed tokens and ring tokens of large norm; two steps, each
    packing the token that leaves the window inside the attention launch."""
    say("value norms: window step")
    H, grp, kb, vb, W = 2, 8, 192, 3, 48
    lens0, steps = (300, 60), 2
    seqs = _seqs([n + steps for n in lens0], H, grp, kb, vb, "both", seed=37)
    nq, S = H * grp, len(lens0)
    cap = 448
    r = run_batch([(K[:n], V[:n], q) for (K, V, q), n in zip(seqs, lens0)], kb, vb, cap, check_attn=False)
    g, off, ogeom, region = r["g"], r["off"], r["ogeom"], kvq.cache_bytes(r["g"])
    cache = torch.zeros(S * region, dtype=torch.uint8, device="cuda")
    win_k = torch.zeros(S, H, W, 128, dtype=torch.float16, device="cuda")
    win_v = torch.zeros_like(win_k)
    for i, ((K, V, _), n) in enumerate(zip(seqs, lens0)):
        npk = n - W
        kvq.quantize_pack(g, K[:npk].cuda(), V[:npk].cuda(), torch.tensor([0], dtype=torch.int64, device="cuda"),
                          torch.tensor([npk], dtype=torch.int32, device="cuda"),
                          torch.tensor([0], dtype=torch.int64, device="cuda"), npk, r["kbits"], r["ksig"], r["vsig"],
                          cache, off[i:i + 1])
        for t in range(npk, n):
            win_k[i, :, t % W] = K[t].cuda()
            win_v[i, :, t % W] = V[t].cuda()
    q = torch.stack([x[2] for x in seqs]).cuda().contiguous()
    out = torch.empty(S, nq, 128, dtype=torch.float32, device="cuda")
    lens = list(lens0)
    for _ in range(steps):
        kn = torch.stack([K[lens[i]] for i, (K, _, _) in enumerate(seqs)]).cuda()
        vn = torch.stack([V[lens[i]] for i, (_, V, _) in enumerate(seqs)]).cuda()
        lens = [n + 1 for n in lens]
        ws = torch.empty(kvq.window_workspace_bytes(g, W, nq, S, max(lens)) // 4, dtype=torch.float32, device="cuda")
        kvq.window_decode_step(g, W, q, kn, vn, win_k, win_v, cache, off,
                               torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens), r["kbits"],
                               r["ksig"], r["vsig"], out, ws)
        oc = cache.cpu().numpy()
        ref = np.stack([oracle.decode_attention_window(
            ogeom, oc[i * region:(i + 1) * region], seqs[i][2].numpy(), lens[i] - W,
            seqs[i][0][lens[i] - W:lens[i]].numpy(), seqs[i][1][lens[i] - W:lens[i]].numpy(), r["ob"], r["osig"],
            r["ovsig"]) for i in range(S)])
        o = out.cpu().numpy()
        assert np.isfinite(o).all()
        say("step worst rel %.2e" % check_attention(o, ref))


@pytest.mark.parametrize("n_split", [1, 3])
def test_prefill_large_value_norms(n_split):
    """Chunked prefill (causal) over values of large norm, one and three key-range splits."""
    say("value norms: prefill split %d" % n_split)
    H, grp, kb, vb = 2, 8, 192, 3
    a, nt = 400, 90
    seqs = _seqs([a + nt], H, grp, kb, vb, "both", seed=41)
    r = run_batch(seqs, kb, vb, 576, check_attn=False)
    g, region = r["g"], kvq.cache_bytes(r["g"])
    wl = synth.Workload("vn", 1, H * grp, H, 1e6, (0,), kb, vb, "decay")
    q = (synth.gen_chunk_queries(wl, 0, 0, a, nt, seed=41).to(torch.float32) * 3).to(torch.float16)
    qd = q[None].cuda().contiguous()
    out = torch.empty(qd.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(kvq.prefill_workspace_bytes(g, H * grp, 1, nt, a + nt, n_split) // 4, 4),
                     dtype=torch.float32, device="cuda")
    kvq.packed_prefill_attn(g, qd, r["cache"], r["off"], torch.tensor([a], dtype=torch.int32, device="cuda"),
                            torch.tensor([nt], dtype=torch.int32, device="cuda"), a + nt, r["kbits"], r["ksig"],
                            r["vsig"], out, ws, n_split=n_split)
    o = out.cpu().numpy()[0]
    assert np.isfinite(o).all()
    ref = oracle.prefill_attention(r["ogeom"], r["oc"][:region], q.numpy(), a, r["ob"], r["osig"], r["ovsig"])
    say("worst rel %.2e" % check_attention(o, ref))


def test_c3_full_size_large_value_norms():
    """One 128K Qwen2.5-3B-shaped layer with value rows of norm 10^2..10^5.6 and
    +-60000 outlier tokens, through the benchmarked fused step (automatic plan)."""
    wl = synth.WORKLOADS["c3"]
    layer = 5
    say("value norms: c3 full-size fused step, layer %d" % layer)
    K, V, _ = synth.gen_layer(wl, 0, layer)
    n = K.shape[0]
    V = big_values(V, 99, "both")
    kn, vn, qn = synth.gen_new_token(wl, 0, layer, n, 0)
    vn = big_values(vn[None], 98, "loguniform")[0]
    qn = (qn.to(torch.float32) * 3).to(torch.float16)
    cap = synth.ceil_to(n + 64, 64)
    r = run_batch([(K, V, qn)], wl.k_budget, wl.v_bits, cap, check_attn=False)
    g, region = r["g"], kvq.cache_bytes(r["g"])
    plan = kvq.decode_plan(g, wl.n_q_heads, 1, cap)
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
    o = out.cpu().numpy()
    assert np.isfinite(o).all()
    say("c3 large norms: worst rel %.2e" % check_attention(o, ref[None]))
