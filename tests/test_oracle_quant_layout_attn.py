"""Pins for the oracle's per-token scale, codes, packed layout and exact attention.

Page: "RoPE-Aware Bit Allocation for KV-Cache Quantization", abstract -- TQ-MSE
quantization at the allocated widths, a packed-cache serving path, and the claim
that Block-GTQ preserves RoPE query-key logits better than uniform TQ-MSE at the
same budget.  Codes are pinned against brute-force nearest-level search, the
layout against hand-derived bytes (tests/golden/layout_v1_tiny.json), attention
against a textbook numpy softmax, and the fidelity claim as a directional gate.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import baselines
from packed_cache_attention_amd import synth

rng = np.random.default_rng(99)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------- per-token scale ----------------

def test_token_scale_properties():
    for _ in range(200):
        x = (rng.standard_normal(128) * 10 ** rng.uniform(-3, 3)).astype(np.float16)
        s = oracle.token_scale(x)
        ref = float(np.sqrt(np.sum(x.astype(np.float64) ** 2)))
        assert abs(s - ref) <= 4e-7 * ref + 1e-30
        # 2^m scaling is exact
        y = (x.astype(np.float32) * 8).astype(np.float16)
        if np.all(np.isfinite(y)) and np.all(y.astype(np.float32) == x.astype(np.float32) * 8):
            assert oracle.token_scale(y) == 8 * s
    # a single non-zero coordinate gives exactly its magnitude
    for v in (np.float16(3.5), np.float16(-1e-7), np.float16(60000)):
        x = np.zeros(128, np.float16)
        x[rng.integers(128)] = v
        assert oracle.token_scale(x) == abs(float(v))
    assert oracle.token_scale(np.zeros(128, np.float16)) == 0.0


def _golden_token(case):
    x = np.zeros(case["d"], np.uint16)
    for k, v in case["coords_fp16_bits"].items():
        if ".." in k:
            a, b = map(int, k.split(".."))
            x[a:b + 1] = v
        else:
            x[int(k)] = v
    return x


def _tree_sum32(sq):
    """Balanced pairwise binary32 sum, pairs (0,1), (2,3), ... at every level."""
    s = np.array(sq, np.float32)
    while len(s) > 1:
        s = (s[0::2] + s[1::2]).astype(np.float32)
    return s[0]


def test_token_scale_tree_order_golden():
    """The per-token scale's summation order decides codes bit for bit; two hand-derived
    tokens (tests/golden/token_scale_tree.json) separate the balanced coordinate-order
    tree from a sequential sum, an exactly rounded sum and a tree that pairs j with
    j + n/2.  The alternatives are evaluated here only to show that each would fail."""
    g = json.load(open(os.path.join(GOLDEN, "token_scale_tree.json")))
    for case in g["cases"]:
        x = _golden_token(case)
        s = np.float32(oracle.token_scale(x))
        assert int(s.view(np.uint32)) == case["expected_scale_bits"], case["name"]
        sq = x.view(np.float16).astype(np.float32) ** 2
        assert np.float32(np.sqrt(_tree_sum32(sq))) == s
        alts = {}
        seq = np.float32(0)
        for v in sq:
            seq = np.float32(seq + v)
        alts["sequential binary32 sum in coordinate order"] = seq
        back = np.float32(0)
        for v in sq[::-1]:
            back = np.float32(back + v)
        alts["sequential sum from the last coordinate down"] = back
        stride = sq.copy()
        while len(stride) > 1:
            stride = (stride[:len(stride) // 2] + stride[len(stride) // 2:]).astype(np.float32)
        alts["balanced tree pairing coordinate j with j + n/2 at each level"] = stride[0]
        alts["exact sum rounded once"] = np.float32(np.sum(sq.astype(np.float64)))
        # each alternative the fixture names gives a different scale
        for name in case["alternatives"]:
            assert np.float32(np.sqrt(alts[name])) != s, (case["name"], name)


# ---------------- codes ----------------

def _brute(y, w):
    lv = oracle.codebook(w)["levels_h"]
    return np.abs(y[:, None] - lv[None, :]).argmin(1)


@pytest.mark.parametrize("w", range(1, 9))
def test_codes_are_nearest_levels(w):
    d = 128
    x = rng.standard_normal((64, d)).astype(np.float16)
    width = np.full(d, w, np.int32)
    sig = np.full(d, 1 / np.sqrt(d), np.float32)
    codes, scale = oracle.encode(x, width, sig)
    y = x.astype(np.float64) / (scale[:, None].astype(np.float64) * float(sig[0]))
    lv = oracle.codebook(w)["levels_h"]
    thr = 0.5 * (lv[1:] + lv[:-1])
    margin = np.min(np.abs(y[..., None] - thr[None, None, :]), axis=-1)
    ok = margin > 1e-5 * np.maximum(np.abs(y), 1e-3)
    ref = _brute(y.reshape(-1), w).reshape(y.shape)
    assert ok.mean() > 0.99
    np.testing.assert_array_equal(codes[ok], ref[ok])
    # sign mirror off thresholds
    codes_neg, _ = oracle.encode((-x.astype(np.float32)).astype(np.float16), width, sig)
    np.testing.assert_array_equal(codes_neg[ok], (1 << w) - 1 - codes[ok])
    # 2^m scaling of the token leaves codes unchanged (scale and thresholds scale exactly)
    codes2, scale2 = oracle.encode((x.astype(np.float32) * 4).astype(np.float16), width, sig)
    np.testing.assert_array_equal(codes2, codes)
    np.testing.assert_array_equal(scale2, scale * 4)


@pytest.mark.parametrize("w", range(1, 9))
def test_dequant_cell_bound(w):
    """A dequantized coordinate is the level of the cell its code names: for an inner
    cell |khat - k| <= s * sigma * (half the gap to the farther neighbouring level),
    and for the two outer cells khat lies on the far side of the one threshold that
    bounds them.  Checked per coordinate against the codebook's own thresholds (the
    midpoints of neighbouring binary16 levels) with the rounding of the binary32
    threshold products as the only slack."""
    d, n = 128, 96
    r = np.random.default_rng(100 + w)
    x = (r.standard_normal((n, d)) * np.exp(r.uniform(-2, 2, (1, d)))).astype(np.float16)
    width = np.full(d, w, np.int32)
    sig = np.exp(r.uniform(-4, 0, d)).astype(np.float32)
    codes, scale = oracle.encode(x, width, sig)
    khat = oracle.dequant(codes, width, sig, scale)
    lv = oracle.codebook(w)["levels_h"]
    thr = np.concatenate([[-np.inf], 0.5 * (lv[1:] + lv[:-1]), [np.inf]])
    unit = scale[:, None].astype(np.float64) * sig[None, :].astype(np.float64)
    xx = x.astype(np.float64)
    c = codes.astype(np.int64)
    slack = 4.0 * 2.0 ** -24 * unit * np.max(np.abs(lv)) + 1e-300
    lo, hi = thr[c], thr[c + 1]
    # the value lies in its cell (up to the threshold products' rounding)
    assert np.all(xx >= unit * lo - slack) and np.all(xx <= unit * hi + slack)
    half = np.maximum(lv[c] - lo, hi - lv[c])
    inner = (c > 0) & (c < (1 << w) - 1)
    assert inner.sum() > n * d // 4 or w == 1
    err = np.abs(khat - xx)
    assert np.all(err[inner] <= (unit * half)[inner] * (1 + 1e-6) + slack[inner])
    # the dequantized value is s * sigma * level, an exact binary16 level times the scales
    np.testing.assert_allclose(khat, unit * lv[c], rtol=1e-15, atol=0)
    top = c == (1 << w) - 1
    assert np.all(khat[top] >= unit[top] * lv[-1] * (1 - 1e-15))
    assert np.all(xx[c == 0] <= (unit * thr[1])[c == 0] + slack[c == 0])


def test_codes_passthrough_and_zero_width():
    d = 128
    x = rng.standard_normal((5, d)).astype(np.float16)
    width = np.array([16] * 64 + [0] * 64, np.int32)
    codes, _ = oracle.encode(x, width, np.ones(d, np.float32))
    np.testing.assert_array_equal(codes[:, :64], x.view(np.uint16)[:, :64])
    assert (codes[:, 64:] == 0).all()
    # zero token: every threshold product is +-0, so all comparisons succeed
    z = np.zeros((1, d), np.float16)
    cz, sz = oracle.encode(z, np.full(d, 3, np.int32), np.full(d, 0.1, np.float32))
    assert sz[0] == 0 and (cz == 7).all()


# ---------------- layout ----------------

def test_layout_golden_bytes():
    g = json.load(open(os.path.join(GOLDEN, "layout_v1_tiny.json")))
    d, kb, vb = g["d"], g["k_budget"], g["v_bits"]
    bits = np.array(g["block_bits"], np.uint8)
    assert oracle.tile_bytes(d, kb, vb) == 1600
    region = np.zeros(g["region_bytes"], np.uint8)
    for tok in g["tokens"]:
        oracle.pack(region, d, g["pairing"], kb, vb, bits, tok["slot"],
                    np.array([tok["kcodes"]], np.uint16), np.array([tok["vcodes"]], np.uint16),
                    np.array([tok["kscale"]], np.float32), np.array([tok["vscale"]], np.float32))
    expect = np.zeros_like(region)
    for off, b in g["nonzero_bytes"].items():
        expect[int(off)] = b
    for off, f in g["floats"].items():
        expect[int(off):int(off) + 4] = np.frombuffer(np.float32(f).tobytes(), np.uint8)
    np.testing.assert_array_equal(region, expect)
    kc, vc, ks, vs = oracle.unpack(region, d, g["pairing"], kb, vb, bits, 65, 1)
    assert kc.tolist() == [g["tokens"][2]["kcodes"]] and vc.tolist() == [g["tokens"][2]["vcodes"]]


def test_k_order_sorted_by_width():
    bits = rng.integers(0, 9, 64).astype(np.uint8)
    order = oracle.k_order(bits, 128, 0)
    p, q = oracle.coord_map(128, 0)
    blk = np.where(order < 64, order, order - 64)
    w = bits[blk]
    assert len(order) == 2 * int((bits > 0).sum())
    assert np.all(np.diff(w.astype(int)) <= 0)
    assert np.all(order[0::2] == p[blk[0::2]]) and np.all(order[1::2] == q[blk[1::2]])


@pytest.mark.parametrize("kb,vb", [(192, 3), (128, 2), (192, 2), (1024, 16), (0, 1), (300, 8)])
def test_pack_roundtrip_and_appends(kb, vb):
    d, H, cap = 128, 2, 192
    geom = oracle.Geometry(H, kb, vb, cap)
    assert geom.tile == 64 * 16 * ((2 * kb + 127) // 128) + 128 * 8 * vb + 512
    n = 150
    k = rng.standard_normal((n, H, d)).astype(np.float16)
    v = rng.standard_normal((n, H, d)).astype(np.float16)
    e = oracle.block_energy(k)
    kbits, ksig = oracle.allocate(e, kb)
    _, vsig = oracle.allocate(oracle.block_energy(v), 64 * vb if vb <= 8 else 1024, oracle.UNIFORM)
    bulk = np.zeros(geom.seq_bytes, np.uint8)
    res = oracle.quantize_pack(geom, bulk, k, v, 0, kbits, ksig, vsig)
    # token-by-token appends (ragged start) give the same bytes
    app = np.zeros_like(bulk)
    oracle.quantize_pack(geom, app, k[:37], v[:37], 0, kbits, ksig, vsig)
    for t in range(37, n):
        oracle.quantize_pack(geom, app, k[t:t + 1], v[t:t + 1], t, kbits, ksig, vsig)
    np.testing.assert_array_equal(app, bulk)
    for h in range(H):
        view = bulk[h * geom.n_tiles * geom.tile:(h + 1) * geom.n_tiles * geom.tile]
        kc, vc, ks, vs = oracle.unpack(view, d, 0, kb, vb, kbits[h], 0, n)
        np.testing.assert_array_equal(kc, res[h][0])
        np.testing.assert_array_equal(vc, res[h][1])
        np.testing.assert_array_equal(ks, res[h][2])


# ---------------- attention ----------------

def _textbook_attention(q, K, V, scale):
    z = (K.astype(np.float64) @ q.astype(np.float64)) * scale
    p = np.exp(z - z.max())
    return (p / p.sum()) @ V.astype(np.float64)


def test_passthrough_attention_is_exact():
    """K16V16: the dequantized cache is the fp16 cache, so attention is textbook attention."""
    H, g, n, cap = 2, 3, 200, 256
    geom = oracle.Geometry(H, 1024, 16, cap)
    k = rng.standard_normal((n, H, 128)).astype(np.float16)
    v = rng.standard_normal((n, H, 128)).astype(np.float16)
    q = rng.standard_normal((H * g, 128)).astype(np.float16)
    kbits, ksig = oracle.allocate(oracle.block_energy(k), 1024)
    _, vsig = oracle.allocate(oracle.block_energy(v), 1024)
    region = np.zeros(geom.seq_bytes, np.uint8)
    oracle.quantize_pack(geom, region, k, v, 0, kbits, ksig, vsig)
    out = oracle.decode_attention(geom, region, q, n, kbits, ksig, vsig)
    for h in range(H * g):
        ref = _textbook_attention(q[h], k[:, h // g], v[:, h // g], 1 / np.sqrt(128))
        np.testing.assert_allclose(out[h], ref, rtol=1e-12, atol=1e-14)
    # logits at 16 bits/dim equal the fp logits: zero logit MAE
    assert baselines.logit_mae(q[:1], k[:, 0], k[:, 0].astype(np.float64)) == 0.0


def test_attention_special_cases():
    H, n, cap = 1, 100, 128
    geom = oracle.Geometry(H, 192, 3, cap)
    k = rng.standard_normal((n, H, 128)).astype(np.float16)
    v = rng.standard_normal((n, H, 128)).astype(np.float16)
    kbits, ksig = oracle.allocate(oracle.block_energy(k), 192)
    _, vsig = oracle.allocate(oracle.block_energy(v), 192, oracle.UNIFORM)
    region = np.zeros(geom.seq_bytes, np.uint8)
    res = oracle.quantize_pack(geom, region, k, v, 0, kbits, ksig, vsig)
    vw = np.full(128, 3, np.int32)
    vhat = oracle.dequant(res[0][1], vw, oracle.per_coord(vsig[0], 128, 0), res[0][3])
    # one token: output is that token's dequantized value
    o1 = oracle.decode_attention(geom, region, rng.standard_normal((1, 128)).astype(np.float16), 1, kbits, ksig, vsig)
    np.testing.assert_allclose(o1[0], vhat[0], rtol=1e-13, atol=1e-15)
    # zero query: uniform softmax, output is the mean of the dequantized values
    o0 = oracle.decode_attention(geom, region, np.zeros((1, 128), np.float16), n, kbits, ksig, vsig)
    np.testing.assert_allclose(o0[0], vhat.mean(0), rtol=1e-12, atol=1e-14)
    # empty sequence: zeros
    oe = oracle.decode_attention(geom, region, np.ones((1, 128), np.float16), 0, kbits, ksig, vsig)
    assert (oe == 0).all()


def test_attention_shift_permutation_and_dominance():
    """Exact attention is unchanged by a constant added to every logit (an extra
    coordinate with q = 1 and khat = C for all tokens), by any reordering of the
    tokens, and returns the value row of a token whose logit exceeds the others' by
    far more than the double exponent range can weigh."""
    r = np.random.default_rng(5)
    n, d = 300, 128
    q = r.standard_normal(d)
    K = r.standard_normal((n, d))
    V = r.standard_normal((n, d))
    sc = 1 / np.sqrt(d)
    o = oracle.attend(q, K, V, sc)
    for C in (-3e4, -7.5, 0.25, 40.0, 3e4):
        q1 = np.concatenate([q, [1.0]])
        K1 = np.concatenate([K, np.full((n, 1), C)], 1)
        V1 = np.concatenate([V, r.standard_normal((n, 1))], 1)
        o1 = oracle.attend(q1, K1, V1, sc)
        np.testing.assert_allclose(o1[:d], o, rtol=1e-11, atol=1e-13)
    perm = r.permutation(n)
    np.testing.assert_allclose(oracle.attend(q, K[perm], V[perm], sc), o, rtol=1e-11, atol=1e-13)
    K2 = K.copy()
    K2[123] = q * 1e4  # logit ~ 1e4 * |q|^2 / sqrt(d), others O(1)
    np.testing.assert_array_equal(oracle.attend(q, K2, V, sc), V[123])
    # the reference -- text book softmax in numpy on the same operands
    z = K @ q * sc
    p = np.exp(z - z.max())
    np.testing.assert_allclose(o, (p / p.sum()) @ V, rtol=1e-12, atol=1e-14)


def test_split_merge_equals_full_attention():
    """Split-K: exact attention of every chunk of a partition of the tokens (empty
    chunks included), merged by the log-sum-exp rule, equals exact attention over all
    tokens; shifting a partial's reference by delta (l, o scaled by 2^-delta) leaves
    the merge unchanged; a row of empty partials merges to 0; one chunk merges to o/l."""
    r = np.random.default_rng(11)
    n, d = 517, 128
    q = r.standard_normal(d)
    K = r.standard_normal((n, d)) * 2.0
    V = r.standard_normal((n, d))
    sc = 1 / np.sqrt(d)
    full = oracle.attend(q, K, V, sc)
    for n_split in (1, 2, 7, 33):
        cuts = np.sort(r.integers(0, n + 1, n_split - 1))
        bounds = np.concatenate([[0], cuts, [n]])
        part = np.zeros((1, n_split, d + 2), np.float64)
        for j in range(n_split):
            a, b = bounds[j], bounds[j + 1]
            m, l_, o = oracle.attend_partial(q, K[a:b], V[a:b], sc)
            if b == a:
                assert m == -np.inf and l_ == 0 and not o.any()
            part[0, j, 0], part[0, j, 1], part[0, j, 2:] = m, l_, o
        # the merge takes binary32 partials, so allow their rounding
        merged = oracle.merge_partials(part.astype(np.float32))[0]
        np.testing.assert_allclose(merged, full, rtol=0, atol=2e-6 * np.abs(full).max())
        shifted = part.copy()
        fin = np.isfinite(shifted[0, :, 0])
        delta = r.uniform(-5, 5, n_split)
        shifted[0, fin, 0] += delta[fin]
        shifted[0, fin, 1:] *= 2.0 ** -delta[fin, None]
        np.testing.assert_allclose(oracle.merge_partials(shifted.astype(np.float32))[0], merged,
                                   rtol=0, atol=2e-6 * np.abs(full).max())
    single = np.zeros((1, 1, d + 2), np.float32)
    single[0, 0, 0], single[0, 0, 1], single[0, 0, 2:] = 3.0, 4.0, np.arange(d)
    np.testing.assert_array_equal(oracle.merge_partials(single)[0], np.arange(d) / 4.0)
    empty = np.zeros((2, 3, d + 2), np.float32)
    empty[:, :, 0] = -np.inf
    assert not oracle.merge_partials(empty).any()


def test_window_attention_pins():
    """fp16 recent window: a window holding every token is textbook attention on the
    fp16 inputs; an empty window is the packed-only attention; with the passthrough
    widths (K16V16) moving tokens between the packed prefix and the window changes
    nothing; a window token enters at its exact value, a packed one dequantized."""
    H, g, n, cap = 2, 3, 150, 192
    k = rng.standard_normal((n, H, 128)).astype(np.float16)
    v = rng.standard_normal((n, H, 128)).astype(np.float16)
    q = rng.standard_normal((H * g, 128)).astype(np.float16)
    sc = 1 / np.sqrt(128)
    geom = oracle.Geometry(H, 192, 3, cap)
    kbits, ksig = oracle.allocate(oracle.block_energy(k), 192)
    _, vsig = oracle.allocate(oracle.block_energy(v), 192, oracle.UNIFORM)
    region = np.zeros(geom.seq_bytes, np.uint8)
    oracle.quantize_pack(geom, region, k, v, 0, kbits, ksig, vsig)
    # every token in the window: no quantization at all
    allw = oracle.decode_attention_window(geom, region, q, 0, k, v, kbits, ksig, vsig)
    for h in range(H * g):
        ref = _textbook_attention(q[h], k[:, h // g], v[:, h // g], sc)
        np.testing.assert_allclose(allw[h], ref, rtol=1e-12, atol=1e-14)
    # empty window: the packed-only attention
    now = oracle.decode_attention_window(geom, region, q, n, k[:0], v[:0], kbits, ksig, vsig)
    np.testing.assert_array_equal(now, oracle.decode_attention(geom, region, q, n, kbits, ksig, vsig))
    # packed prefix + window differs from all-packed only through the window tokens'
    # quantization error: closer to the exact attention than the all-packed result
    mix = oracle.decode_attention_window(geom, region, q, n - 40, k[n - 40:], v[n - 40:], kbits, ksig, vsig)
    allp = oracle.decode_attention(geom, region, q, n, kbits, ksig, vsig)
    assert np.abs(mix - allw).max() < np.abs(allp - allw).max()
    # passthrough widths: where a token sits does not matter
    gp = oracle.Geometry(H, 1024, 16, cap)
    kb16, ks16 = oracle.allocate(oracle.block_energy(k), 1024)
    _, vs16 = oracle.allocate(oracle.block_energy(v), 1024)
    reg16 = np.zeros(gp.seq_bytes, np.uint8)
    oracle.quantize_pack(gp, reg16, k, v, 0, kb16, ks16, vs16)
    for split in (0, 1, 64, 149, 150):
        o = oracle.decode_attention_window(gp, reg16, q, split, k[split:], v[split:], kb16, ks16, vs16)
        np.testing.assert_allclose(o, allw, rtol=1e-12, atol=1e-14)


def test_prefill_attention_pins():
    """Chunked prefill (causal): with the passthrough widths (K16V16) every row is
    textbook causal attention on the fp16 inputs (the mask admits exactly the slots
    up to the query's own position); with packed widths row j is the decode
    attention at length q_start + j + 1; the chunk's first query at position 0 sees
    only slot 0 (output = its dequantized value); a zero query averages the
    dequantized values it sees; slots past the chunk's last query never matter."""
    H, g, n, cap = 2, 3, 150, 192
    k = rng.standard_normal((n, H, 128)).astype(np.float16)
    v = rng.standard_normal((n, H, 128)).astype(np.float16)
    sc = 1 / np.sqrt(128)
    # passthrough: textbook causal attention, chunk in the middle and at the start
    gp = oracle.Geometry(H, 1024, 16, cap)
    kb16, ks16 = oracle.allocate(oracle.block_energy(k), 1024)
    _, vs16 = oracle.allocate(oracle.block_energy(v), 1024)
    reg16 = np.zeros(gp.seq_bytes, np.uint8)
    oracle.quantize_pack(gp, reg16, k, v, 0, kb16, ks16, vs16)
    for q0, nt in ((70, 30), (0, 9)):
        q = rng.standard_normal((nt, H * g, 128)).astype(np.float16)
        o = oracle.prefill_attention(gp, reg16, q, q0, kb16, ks16, vs16)
        for j in range(nt):
            for h in range(H * g):
                ref = _textbook_attention(q[j, h], k[:q0 + j + 1, h // g], v[:q0 + j + 1, h // g], sc)
                np.testing.assert_allclose(o[j, h], ref, rtol=1e-12, atol=1e-14)
    # packed widths: rows are decode attention at their own lengths
    geom = oracle.Geometry(H, 192, 3, cap)
    kbits, ksig = oracle.allocate(oracle.block_energy(k), 192)
    _, vsig = oracle.allocate(oracle.block_energy(v), 192, oracle.UNIFORM)
    region = np.zeros(geom.seq_bytes, np.uint8)
    res = oracle.quantize_pack(geom, region, k, v, 0, kbits, ksig, vsig)
    q0, nt = 100, 50
    q = rng.standard_normal((nt, H * g, 128)).astype(np.float16)
    o = oracle.prefill_attention(geom, region, q, q0, kbits, ksig, vsig)
    for j in (0, 1, 17, 49):
        np.testing.assert_array_equal(o[j], oracle.decode_attention(geom, region, q[j], q0 + j + 1,
                                                                    kbits, ksig, vsig))
    # position 0 sees slot 0 only; a zero query is the mean of what it sees
    vw = np.full(128, 3, np.int32)
    vhat = [oracle.dequant(res[h][1], vw, oracle.per_coord(vsig[h], 128, 0), res[h][3]) for h in range(H)]
    qz = rng.standard_normal((4, H * g, 128)).astype(np.float16)
    qz[2] = 0
    oz = oracle.prefill_attention(geom, region, qz, 0, kbits, ksig, vsig)
    for h in range(H * g):
        np.testing.assert_allclose(oz[0, h], vhat[h // g][0], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(oz[2, h], vhat[h // g][:3].mean(0), rtol=1e-12, atol=1e-14)
    # slots after the chunk's last query are never read (chunk ends at slot 127)
    q0, nt = 70, 58
    q = rng.standard_normal((nt, H * g, 128)).astype(np.float16)
    o = oracle.prefill_attention(geom, region, q, q0, kbits, ksig, vsig)
    spoiled = region.copy()
    view_len = geom.n_tiles * geom.tile
    for h in range(H):
        t = spoiled[h * view_len:(h + 1) * view_len].reshape(geom.n_tiles, geom.tile)
        t[2, :] = 0xA5  # tile 2 = slots 128..191
    o2 = oracle.prefill_attention(geom, spoiled, q, q0, kbits, ksig, vsig)
    np.testing.assert_array_equal(o2, o)


# (config, tokens, [(sequence, layer, KV head), ...]): every seeded config, sampled
# layers and heads (the model-shaped configs draw each (sequence, layer, head) from a
# stream of its own; the 512K config shares the 128K one's streams, so it is sampled
# at other layers)
GATE_CASES = [
    ("c1", 1024, [(0, 0, 0)]),
    ("c2", 8192, [(0, 0, 0), (0, 0, 5)]),
    ("c3", 4096, [(0, 0, 0), (0, 17, 1), (0, 35, 0)]),
    ("c4", 8192, [(0, 5, 1), (0, 29, 0)]),
    ("c5", 4096, [(3, 0, 0), (11, 27, 3), (7, 13, 2)]),
]


@pytest.mark.parametrize("cfg,n,units", GATE_CASES)
def test_fidelity_gate_beats_uniform(cfg, n, units):
    """Block-GTQ's query-key logit MAE is no worse than either uniform baseline at the
    same K budget (the page's per-layer comparison against uniform TQ-MSE), on sampled
    layers and heads of every seeded config."""
    wl = synth.WORKLOADS[cfg]
    for seq, layer, h in units:
        k, _, q = synth.gen_head(wl, seq, layer, h, n)
        r = baselines.mae_report(q.numpy(), k.numpy(), wl.k_budget)
        assert r["blockgtq"] <= r["u_same"] and r["blockgtq"] <= r["u_rot"], (cfg, seq, layer, h, r)
        assert r["blockgtq"] < 0.7 * min(r["u_same"], r["u_rot"]), (cfg, seq, layer, h, r)
