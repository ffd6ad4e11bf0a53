"""The decode step replayed from a HIP graph, as the throughput figures time it.

Per layer the step is either one `kvq_decode_step` call or the split-phase pair
`kvq_decode_step_partials` + `kvq_merge_partials`, with the sequences' lengths advanced
on the device, all captured once; the fp16-window step (`kvq_window_decode_step`) the same
way.  Each replay runs after eager work of the program (the next tokens copied into
the captured input buffers, an eager run of the same step on a second copy of the
state, synchronisations), and every replay is compared with that eager run: packed
bytes, ring rows and outputs identical.  At the end the packed bytes equal the
oracle's quantization of every token and the outputs its attention within 2e-3 per
head (the parity bar of "RoPE-Aware Bit Allocation for KV-Cache Quantization"'s
packed serving path as read here)."""
import numpy as np
import pytest
import torch

import oracle
from packed_cache_attention_amd import kvq, synth

from pipeline import check_attention, run_batch, say

pytestmark = pytest.mark.gpu

STEPS = 5


def _layers(L, H, grp, kb, vb, n0, extra, cap):
    """Per layer: the sequences' tokens (initial + extra) and the prefill state from the
    initial tokens (allocation and packed bytes checked against the oracle inside)."""
    wl = synth.Workload("graph", L, H * grp, H, 1e6, (0,), kb, vb, "decay")
    out = []
    for l in range(L):
        seqs = [synth.gen_layer(wl.with_lens([n + extra]), i, l, n_tok=n + extra, seed=61) for i, n in enumerate(n0)]
        r = run_batch([(K[:n], V[:n], q) for (K, V, q), n in zip(seqs, n0)], kb, vb, cap, check_attn=False)
        out.append((seqs, r))
    return out


@pytest.mark.parametrize("fused", [True, False], ids=["decode_step", "partials+merge"])
def test_graph_replays_of_the_decode_step_equal_eager_steps(fused):
    L, H, grp, kb, vb = 2, 2, 8, 192, 3
    n0 = [700, 63, 129]
    S, nq = len(n0), H * grp
    cap = 64 * ((max(n0) + STEPS + 63) // 64 + 1)
    say("graph (%s): %d layers, lengths %s, %d replays" % ("decode_step" if fused else "partials+merge", L, n0,
                                                         STEPS))
    layers = _layers(L, H, grp, kb, vb, n0, STEPS, cap)
    g, off = layers[0][1]["g"], layers[0][1]["off"]
    region = kvq.cache_bytes(g)
    plan = kvq.decode_plan(g, nq, S, cap)
    n_split = plan["n_split"]

    def state():
        return {"cache": [r["cache"].clone() for _, r in layers],
                "cur": torch.tensor(n0, dtype=torch.int64, device="cuda"),
                "seq_len": torch.tensor([n + 1 for n in n0], dtype=torch.int32, device="cuda"),
                "part": torch.empty(L, plan["workspace"] // 4, dtype=torch.float32, device="cuda"),
                "out": torch.full((L, S, nq, 128), float("nan"), dtype=torch.float32, device="cuda")}

    qs = [torch.stack([x[2] for x in seqs]).cuda().contiguous() for seqs, _ in layers]
    knew = torch.empty(L, S, H, 128, dtype=torch.float16, device="cuda")
    vnew = torch.empty_like(knew)

    def step(st):
        for l, (_, r) in enumerate(layers):
            if fused:
                kvq.decode_step(g, qs[l], knew[l], vnew[l], st["cache"][l], off, st["seq_len"], cap, r["kbits"],
                                r["ksig"], r["vsig"], st["out"][l], st["part"][l])
                continue
            kvq.decode_step_partials(g, qs[l], knew[l], vnew[l], st["cache"][l], off, st["seq_len"], cap, r["kbits"],
                                     r["ksig"], r["vsig"], st["part"][l])
            kvq.merge_partials(S, nq, n_split, st["part"][l], st["out"][l])
        st["cur"].add_(1)
        st["seq_len"].add_(1)

    def load_tokens(t):
        for l, (seqs, _) in enumerate(layers):
            knew[l] = torch.stack([K[n0[i] + t] for i, (K, _, _) in enumerate(seqs)]).cuda()
            vnew[l] = torch.stack([V[n0[i] + t] for i, (_, V, _) in enumerate(seqs)]).cuda()

    sg, se = state(), state()
    torch.cuda.synchronize()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(graph, stream=s_cap):
            step(sg)
    torch.cuda.current_stream().wait_stream(s_cap)
    torch.cuda.synchronize()
    for t in range(STEPS):
        load_tokens(t)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(se)
        torch.cuda.synchronize()
        for l in range(L):
            np.testing.assert_array_equal(sg["cache"][l].cpu().numpy(), se["cache"][l].cpu().numpy())
        np.testing.assert_array_equal(sg["out"].cpu().numpy(), se["out"].cpu().numpy())
        assert torch.equal(sg["seq_len"], se["seq_len"]) and torch.equal(sg["cur"], se["cur"])
        say("graph replay %d equals the eager step" % t)
    # the oracle: every token quantized and packed, attention over all of them
    for l, (seqs, r) in enumerate(layers):
        oc = np.zeros(S * region, np.uint8)
        for i, (K, V, _) in enumerate(seqs):
            oracle.quantize_pack(r["ogeom"], oc[i * region:(i + 1) * region], K.numpy(), V.numpy(), 0, r["ob"],
                                 r["osig"], r["ovsig"])
        np.testing.assert_array_equal(sg["cache"][l].cpu().numpy(), oc)
        ref = np.stack([oracle.decode_attention(r["ogeom"], oc[i * region:(i + 1) * region], seqs[i][2].numpy(),
                                                n0[i] + STEPS, r["ob"], r["osig"], r["ovsig"]) for i in range(S)])
        check_attention(sg["out"][l].cpu().numpy(), ref)


def test_graph_replays_of_the_window_step_equal_eager_steps():
    L, H, grp, kb, vb, W = 2, 2, 8, 192, 3, 64
    n0 = [300, 40]
    S, nq = len(n0), H * grp
    cap = 64 * ((max(n0) + STEPS + 63) // 64 + 1)
    say("graph window: %d layers, W %d, lengths %s, %d replays" % (L, W, n0, STEPS))
    layers = _layers(L, H, grp, kb, vb, n0, STEPS, cap)
    g, off = layers[0][1]["g"], layers[0][1]["off"]
    region = kvq.cache_bytes(g)
    max_len = max(n0) + STEPS
    ws_words = kvq.window_workspace_bytes(g, W, nq, S, max_len) // 4

    def state():
        st = {"cache": [], "wk": [], "wv": [],
              "seq_len": torch.tensor(n0, dtype=torch.int32, device="cuda"),
              "ws": torch.empty(L, ws_words, dtype=torch.float32, device="cuda"),
              "out": torch.full((L, S, nq, 128), float("nan"), dtype=torch.float32, device="cuda")}
        for seqs, r in layers:
            cache = torch.zeros(S * region, dtype=torch.uint8, device="cuda")
            wk = torch.zeros(S, H, W, 128, dtype=torch.float16, device="cuda")
            wv = torch.zeros_like(wk)
            for i, ((K, V, _), n) in enumerate(zip(seqs, n0)):
                npk = max(n - W, 0)
                if npk > 0:
                    kvq.quantize_pack(g, K[:npk].cuda(), V[:npk].cuda(),
                                      torch.tensor([0], dtype=torch.int64, device="cuda"),
                                      torch.tensor([npk], dtype=torch.int32, device="cuda"),
                                      torch.tensor([0], dtype=torch.int64, device="cuda"), npk, r["kbits"],
                                      r["ksig"], r["vsig"], cache, off[i:i + 1])
                for t in range(npk, n):
                    wk[i, :, t % W] = K[t].cuda()
                    wv[i, :, t % W] = V[t].cuda()
            st["cache"].append(cache)
            st["wk"].append(wk)
            st["wv"].append(wv)
        return st

    qs = [torch.stack([x[2] for x in seqs]).cuda().contiguous() for seqs, _ in layers]
    knew = torch.empty(L, S, H, 128, dtype=torch.float16, device="cuda")
    vnew = torch.empty_like(knew)

    def step(st):
        st["seq_len"].add_(1)
        for l, (_, r) in enumerate(layers):
            kvq.window_decode_step(g, W, qs[l], knew[l], vnew[l], st["wk"][l], st["wv"][l], st["cache"][l], off,
                                   st["seq_len"], max_len, r["kbits"], r["ksig"], r["vsig"], st["out"][l],
                                   st["ws"][l])

    sg, se = state(), state()
    torch.cuda.synchronize()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(graph, stream=s_cap):
            step(sg)
    torch.cuda.current_stream().wait_stream(s_cap)
    torch.cuda.synchronize()
    for t in range(STEPS):
        for l, (seqs, _) in enumerate(layers):
            knew[l] = torch.stack([K[n0[i] + t] for i, (K, _, _) in enumerate(seqs)]).cuda()
            vnew[l] = torch.stack([V[n0[i] + t] for i, (_, V, _) in enumerate(seqs)]).cuda()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(se)
        torch.cuda.synchronize()
        for l in range(L):
            np.testing.assert_array_equal(sg["cache"][l].cpu().numpy(), se["cache"][l].cpu().numpy())
            assert torch.equal(sg["wk"][l], se["wk"][l]) and torch.equal(sg["wv"][l], se["wv"][l])
        np.testing.assert_array_equal(sg["out"].cpu().numpy(), se["out"].cpu().numpy())
        say("graph window replay %d equals the eager step" % t)
    lens = [n + STEPS for n in n0]
    for l, (seqs, r) in enumerate(layers):
        oc = np.zeros(S * region, np.uint8)
        for i, (K, V, _) in enumerate(seqs):
            npk = max(lens[i] - W, 0)
            if npk > 0:
                oracle.quantize_pack(r["ogeom"], oc[i * region:(i + 1) * region], K[:npk].numpy(), V[:npk].numpy(),
                                     0, r["ob"], r["osig"], r["ovsig"])
        np.testing.assert_array_equal(sg["cache"][l].cpu().numpy(), oc)
        ref = np.stack([oracle.decode_attention_window(
            r["ogeom"], oc[i * region:(i + 1) * region], seqs[i][2].numpy(), max(lens[i] - W, 0),
            seqs[i][0][max(lens[i] - W, 0):lens[i]].numpy(), seqs[i][1][max(lens[i] - W, 0):lens[i]].numpy(),
            r["ob"], r["osig"], r["ovsig"]) for i in range(S)])
        check_attention(sg["out"][l].cpu().numpy(), ref)
