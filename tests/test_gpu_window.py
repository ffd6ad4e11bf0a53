"""GPU parity for the fp16 recent-window variant ("RoPE-Aware Bit Allocation for
KV-Cache Quantization": the recent-key buffer its reasoning evaluation goes
without).  The newest W tokens stay binary16 in a ring, the rest are packed; every
step packs the token leaving the window inside the attention launch and writes the
new one into the ring.  Checked against the oracle: packed bytes bit for bit, ring
rows exactly, attention within 2e-3 per head, over ragged batches whose sequences
start inside the window and cross it, windows of 1..128 tokens, both kernels."""
import numpy as np
import pytest
import torch

import oracle
from packed_cache_attention_amd import kvq, synth

from pipeline import check_attention, run_batch, say

pytestmark = pytest.mark.gpu

CASES = [
    # name, H_kv, group, k_budget, v_bits, window, initial lengths, steps, kernel
    ("k3v3-w64-mfma", 2, 8, 192, 3, 64, (150, 40), 30, kvq.DECODE_AUTO),
    ("k3v3-w64-generic", 2, 8, 192, 3, 64, (150, 40), 30, kvq.DECODE_GENERIC),
    ("k2v2-w100", 2, 4, 128, 2, 100, (300, 99), 5, kvq.DECODE_AUTO),
    ("kodd-v5-w37", 1, 3, 131, 5, 37, (90, 3), 40, kvq.DECODE_AUTO),
    ("konly-v16-w64", 2, 2, 192, 16, 64, (130, 64), 3, kvq.DECODE_AUTO),
    ("konly-v16-g8-w32", 2, 8, 192, 16, 32, (200, 31), 10, kvq.DECODE_AUTO),
    ("k3v2-gqa7-w128", 2, 7, 192, 2, 128, (200, 129), 4, kvq.DECODE_AUTO),
    ("k3v3-w1", 1, 4, 192, 3, 1, (70, 1), 3, kvq.DECODE_AUTO),
]


def _random_cases(n):
    # seeded random valid cases: heads, group, budgets, window, ragged starts, steps, kernel
    r = np.random.default_rng(77)
    out = []
    for i in range(n):
        H = int(r.integers(1, 4))
        grp = int(r.choice([1, 2, 4, 7, 8, 16]))
        kb = int(r.integers(0, 257))
        vb = 16 if r.random() < 0.2 else int(r.integers(1, 9))
        W = int(r.integers(1, 200))
        n0 = tuple(int(x) for x in r.integers(1, 400, int(r.integers(1, 4))))
        steps = int(r.integers(1, 4))
        kernel = kvq.DECODE_GENERIC if r.random() < 0.3 else kvq.DECODE_AUTO
        out.append(("random%d" % i, H, grp, kb, vb, W, n0, steps, kernel))
    return out


CASES += _random_cases(6)


def _window_tokens(X, n, W):
    """Tokens [max(n - W, 0), n) of X [N, H, d] (the window, in sequence order)."""
    return X[max(n - W, 0):n]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_window_steps_match_oracle(case):
    name, H, grp, kb, vb, W, n0, steps, kernel = case
    say("window %s" % name)
    nq, S = H * grp, len(n0)
    wl = synth.Workload("win-" + name, 1, nq, H, 1e6, (0,), kb, vb, "decay")
    seqs = [synth.gen_layer(wl.with_lens([n + steps]), i, 0, n_tok=n + steps, seed=31 + i) for i, n in enumerate(n0)]
    cap = 64 * ((max(n0) + steps + 63) // 64 + 1)
    # allocation (and the oracle's) from the initial tokens; the packed cache is rebuilt below
    r = run_batch([(K[:n], V[:n], q) for (K, V, q), n in zip(seqs, n0)], kb, vb, cap, check_attn=False)
    g, off, ogeom = r["g"], r["off"], r["ogeom"]
    region = kvq.cache_bytes(g)
    cache = torch.zeros(S * region, dtype=torch.uint8, device="cuda")
    win_k = torch.zeros(S, H, W, 128, dtype=torch.float16, device="cuda")
    win_v = torch.zeros_like(win_k)
    for i, ((K, V, _), n) in enumerate(zip(seqs, n0)):
        npk = max(n - W, 0)
        if npk > 0:
            kvq.quantize_pack(g, K[:npk].cuda(), V[:npk].cuda(), torch.tensor([0], dtype=torch.int64, device="cuda"),
                              torch.tensor([npk], dtype=torch.int32, device="cuda"),
                              torch.tensor([0], dtype=torch.int64, device="cuda"), npk, r["kbits"], r["ksig"],
                              r["vsig"], cache, off[i:i + 1])
        for t in range(npk, n):
            win_k[i, :, t % W] = K[t].cuda()
            win_v[i, :, t % W] = V[t].cuda()
    q = torch.stack([x[2] for x in seqs]).cuda().contiguous()

    def ws_for(max_len):
        return torch.empty(kvq.window_workspace_bytes(g, W, nq, S, max_len, kernel) // 4, dtype=torch.float32,
                           device="cuda")

    def ref_attention(lens):
        oc = cache.cpu().numpy()
        return np.stack([oracle.decode_attention_window(
            ogeom, oc[i * region:(i + 1) * region], seqs[i][2].numpy(), max(lens[i] - W, 0),
            _window_tokens(seqs[i][0], lens[i], W).numpy(), _window_tokens(seqs[i][1], lens[i], W).numpy(),
            r["ob"], r["osig"], r["ovsig"]) for i in range(S)])

    # attention alone over the prefill state
    lens = list(n0)
    out = torch.empty(S, nq, 128, dtype=torch.float32, device="cuda")
    kvq.window_decode_attn(g, W, q, win_k, win_v, cache, off, torch.tensor(lens, dtype=torch.int32, device="cuda"),
                           max(lens), r["kbits"], r["ksig"], r["vsig"], out, ws_for(max(lens)), kernel=kernel)
    check_attention(out.cpu().numpy(), ref_attention(lens))
    # steps
    for st in range(steps):
        kn = torch.stack([K[lens[i]] for i, (K, _, _) in enumerate(seqs)]).cuda()
        vn = torch.stack([V[lens[i]] for i, (_, V, _) in enumerate(seqs)]).cuda()
        lens = [n + 1 for n in lens]
        kvq.window_decode_step(g, W, q, kn, vn, win_k, win_v, cache, off,
                               torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens), r["kbits"],
                               r["ksig"], r["vsig"], out, ws_for(max(lens)), kernel=kernel)
        check_attention(out.cpu().numpy(), ref_attention(lens))
    # packed bytes: the oracle's quantization of tokens [0, n - W); ring rows exact
    oc = np.zeros(S * region, np.uint8)
    for i, (K, V, _) in enumerate(seqs):
        npk = max(lens[i] - W, 0)
        if npk > 0:
            oracle.quantize_pack(ogeom, oc[i * region:(i + 1) * region], K[:npk].numpy(), V[:npk].numpy(), 0,
                                 r["ob"], r["osig"], r["ovsig"])
    np.testing.assert_array_equal(cache.cpu().numpy(), oc)
    wk, wv = win_k.cpu(), win_v.cpu()
    for i, (K, V, _) in enumerate(seqs):
        for t in range(max(lens[i] - W, 0), lens[i]):
            assert torch.equal(wk[i, :, t % W], K[t]) and torch.equal(wv[i, :, t % W], V[t])


def test_c3_full_size_window_step_as_benchmarked():
    """The window step the benchmark times, at its size: one 128K Qwen2.5-3B-shaped layer
    with W = 128 (131072 tokens: the first 130944 packed, the newest 128 in the ring),
    one kvq_window_decode_step in the automatic plan with max_len = capacity.  The token
    leaving the window is packed inside the attention launch (bytes against the
    oracle's packing), the new token takes its ring row (exact), and the output matches
    the oracle's attention over the packed prefix and the fp16 window."""
    wl = synth.WORKLOADS["c3"]
    layer, W = 5, 128
    say("c3 full-size window step, layer %d, W %d" % (layer, W))
    K, V, _ = synth.gen_layer(wl, 0, layer)
    n = K.shape[0]
    kn, vn, qn = synth.gen_new_token(wl, 0, layer, n, 0)
    cap = synth.ceil_to(n + 64, 64)
    npk = n - W
    r = run_batch([(K[:npk], V[:npk], qn)], wl.k_budget, wl.v_bits, cap, check_attn=False)
    g, region, H = r["g"], kvq.cache_bytes(r["g"]), wl.n_kv_heads
    win_k = torch.empty(1, H, W, 128, dtype=torch.float16)
    win_v = torch.empty_like(win_k)
    for t in range(npk, n):
        win_k[0, :, t % W] = K[t]
        win_v[0, :, t % W] = V[t]
    win_k, win_v = win_k.cuda(), win_v.cuda()
    ws = torch.empty(kvq.window_workspace_bytes(g, W, wl.n_q_heads, 1, cap) // 4 + 4, dtype=torch.float32,
                     device="cuda")
    out = torch.empty(1, wl.n_q_heads, 128, dtype=torch.float32, device="cuda")
    kvq.window_decode_step(g, W, qn[None].cuda().contiguous(), kn[None].cuda().contiguous(),
                           vn[None].cuda().contiguous(), win_k, win_v, r["cache"], r["off"],
                           torch.tensor([n + 1], dtype=torch.int32, device="cuda"), cap, r["kbits"], r["ksig"],
                           r["vsig"], out, ws)
    # the token leaving the window (position n - W) packed at its slot
    oc = r["oc"].copy()
    oracle.quantize_pack(r["ogeom"], oc[:region], K[npk:npk + 1].numpy(), V[npk:npk + 1].numpy(), npk, r["ob"],
                         r["osig"], r["ovsig"])
    np.testing.assert_array_equal(r["cache"].cpu().numpy(), oc)
    # the new token in the ring row the leaving token held; the other rows untouched
    wk, wv = win_k.cpu(), win_v.cpu()
    assert torch.equal(wk[0, :, n % W], kn) and torch.equal(wv[0, :, n % W], vn)
    for t in range(npk + 1, n):
        assert torch.equal(wk[0, :, t % W], K[t]) and torch.equal(wv[0, :, t % W], V[t])
    # attention: packed prefix [0, n - W], fp16 window [n - W + 1, n]
    kw = torch.cat([K[npk + 1:n], kn[None]]).numpy()
    vw = torch.cat([V[npk + 1:n], vn[None]]).numpy()
    ref = oracle.decode_attention_window(r["ogeom"], oc[:region], qn.numpy(), npk + 1, kw, vw, r["ob"], r["osig"],
                                         r["ovsig"])
    say("c3 window step: bytes and ring ok, attention worst rel %.2e" % check_attention(out.cpu().numpy(), ref[None]))
