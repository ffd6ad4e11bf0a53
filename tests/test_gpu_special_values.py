"""Quantize + pack of rows holding binary16 special values -- subnormals, signed zeros,
the largest finite values, tiny normals, an all-zero row and a row of 65504s -- through the
bulk kernel, the few-token append kernel and the decode step's append, against the oracle
byte for byte (energies, widths and scales too).  The code rule of "RoPE-Aware Bit
Allocation for KV-Cache Quantization" (TQ-MSE codes at the allocated widths, as read here)
must hold for every finite binary16 input, the token norm included."""
import numpy as np
import pytest
import torch

import oracle
from packed_cache_attention_amd import kvq

from pipeline import run_batch, say

pytestmark = pytest.mark.gpu

SPECIAL = [6e-8, -6e-8, 0.0, -0.0, 65504.0, -65504.0, 1e-5, -3e-6, 6.1e-5, -6.1e-5, 2.0, -1.0, 1e-7, 300.0]

# (name, KV heads, K budget, V bits, pairing)
CASES = [("k3v3", 2, 192, 3, 0), ("k8v8", 1, 512, 8, 0), ("k0v1", 2, 0, 1, 0), ("k2v2-il", 2, 128, 2, 1),
         ("k5v4", 1, 320, 4, 0), ("konly-v16", 1, 192, 16, 0)]


def _rows(n, H, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, H, 128, generator=g, dtype=torch.float64) * 3.0
    flat = x.view(-1)
    r = np.random.default_rng(seed)
    idx = torch.from_numpy(r.choice(flat.numel(), flat.numel() // 20, replace=False))
    flat[idx] = torch.tensor(r.choice(SPECIAL, len(idx)), dtype=torch.float64)
    x[1] = 0.0                  # an all-zero row (norm 0)
    x[2, :, ::2] = 65504.0      # the largest finite values
    x[2, :, 1::2] = -65504.0
    x[3] = 6e-8                 # only subnormals
    return x.to(torch.float16)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_special_values_bulk_and_append(case):
    name, H, kb, vb, pairing = case
    say("special values %s" % name)
    n0, n1 = 70, 9
    K, V = _rows(n0 + n1, H, seed=3), _rows(n0 + n1, H, seed=4)
    # the last rows repeat the special rows so the append path sees them too
    K[n0:n0 + 4] = K[0:4]
    V[n0:n0 + 4] = V[0:4]
    q = torch.zeros(8, 128, dtype=torch.float16)
    r = run_batch([(K[:n0], V[:n0], q)], kb, vb, 128, pairing=pairing, check_attn=False)
    g, cache, off = r["g"], r["cache"], r["off"]
    cache2 = cache.clone()  # the bulk state, for the decode step's appends below
    rows, vrows = K.cuda(), V.cuda()
    done = n0
    while done < n0 + n1:
        c = min(3, n0 + n1 - done)
        kvq.quantize_pack(g, rows, vrows, torch.tensor([done], dtype=torch.int64, device="cuda"),
                          torch.tensor([c], dtype=torch.int32, device="cuda"),
                          torch.tensor([done], dtype=torch.int64, device="cuda"), 4, r["kbits"], r["ksig"], r["vsig"],
                          cache, off)
        done += c
    region = kvq.cache_bytes(g)
    oc = np.zeros(region, np.uint8)
    oracle.quantize_pack(r["ogeom"], oc, K.numpy(), V.numpy(), 0, r["ob"], r["osig"], r["ovsig"])
    np.testing.assert_array_equal(cache.cpu().numpy(), oc)
    # the decode step's own append (inside the attention launch where the kernel allows),
    # one token per step from the same bulk state
    nq = q.shape[0]
    qs = torch.zeros(1, nq, 128, dtype=torch.float16, device="cuda")
    ws = torch.empty(kvq.decode_workspace_bytes(g, nq, 1, 128) // 4, dtype=torch.float32, device="cuda")
    out = torch.empty(1, nq, 128, dtype=torch.float32, device="cuda")
    for t in range(n0, n0 + n1):
        kvq.decode_step(g, qs, rows[t:t + 1].contiguous(), vrows[t:t + 1].contiguous(), cache2, off,
                        torch.tensor([t + 1], dtype=torch.int32, device="cuda"), 128, r["kbits"], r["ksig"],
                        r["vsig"], out, ws)
    np.testing.assert_array_equal(cache2.cpu().numpy(), oc)
