"""GPU parity of the split-K log-sum-exp merge (kvq_merge_partials) on its own, against
the oracle's fp64 merge of the same binary32 partials: seeded partials with
references spread over +-60 (log2 units), empty chunks (m = -inf, l = 0, o = 0),
whole rows of empty chunks (output exactly 0), and split counts on both sides of the
small-merge limit (16) and beyond one pass of the large one (512)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from packed_cache_attention_amd import kvq

from pipeline import check_attention, say

pytestmark = pytest.mark.gpu


def _partials(rows, n_split, seed):
    r = np.random.default_rng(seed)
    p = np.zeros((rows, n_split, 130), np.float32)
    p[:, :, 0] = r.normal(0, 20, (rows, n_split))
    p[:, :, 1] = np.exp(r.uniform(-3, 8, (rows, n_split)))
    p[:, :, 2:] = r.standard_normal((rows, n_split, 128)) * p[:, :, 1:2] * 0.3
    empty = r.random((rows, n_split)) < 0.2
    p[empty, 0] = -np.inf
    p[empty, 1:] = 0
    p[-1, :, 0] = -np.inf  # a row that attended nothing
    p[-1, :, 1:] = 0
    return p


@pytest.mark.parametrize("n_split", [1, 2, 7, 16, 17, 100, 257, 512, 700])
def test_merge_matches_oracle(n_split):
    rows = 37
    say("merge n_split %d" % n_split)
    p = _partials(rows, n_split, 1000 + n_split)
    out = torch.full((rows, 128), float("nan"), dtype=torch.float32, device="cuda")
    kvq.merge_partials(1, rows, n_split, torch.from_numpy(p).cuda(), out)
    o = out.cpu().numpy()
    ref = oracle.merge_partials(p)
    assert (o[-1] == 0).all()
    worst = check_attention(o, ref, tol=1e-5)
    say("merge n_split %d worst rel %.2e" % (n_split, worst))


def test_token_scale_golden_on_gpu():
    """The hand-derived tokens of tests/golden/token_scale_tree.json, quantized by the
    library as keys and as values: the stored binary32 scales carry the fixture's bits."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "token_scale_tree.json")))
    rows = []
    for case in g["cases"]:
        x = np.zeros(case["d"], np.uint16)
        for k, v in case["coords_fp16_bits"].items():
            if ".." in k:
                a, b = map(int, k.split(".."))
                x[a:b + 1] = v
            else:
                x[int(k)] = v
        rows.append(x)
    X = torch.from_numpy(np.stack(rows).view(np.float16)).reshape(len(rows), 1, 128)
    geo = kvq.geom(1, 192, 3, 64)
    kb = torch.full((1, 64), 3, dtype=torch.uint8, device="cuda")
    sig = torch.full((1, 64), 0.1, dtype=torch.float32, device="cuda")
    cache = torch.zeros(kvq.cache_bytes(geo), dtype=torch.uint8, device="cuda")
    n = len(rows)
    z64 = torch.zeros(1, dtype=torch.int64, device="cuda")
    kvq.quantize_pack(geo, X.cuda(), X.cuda(), z64, torch.tensor([n], dtype=torch.int32, device="cuda"), z64, n,
                      kb, sig, sig, cache, z64)
    tb = kvq.tile_bytes(geo)
    scl = cache.cpu().numpy()[tb - 512:tb].view(np.uint32)
    for i, case in enumerate(g["cases"]):
        assert scl[i] == case["expected_scale_bits"], case["name"]
        assert scl[64 + i] == case["expected_scale_bits"], case["name"]
