"""Shared helpers for the GPU parity tests: run one batch of sequences through the
HIP library (via the C-ABI binding) and through the CPU oracle, stage by stage.

Stage outputs compared: block energies, widths and scales (bit-exact), packed
cache bytes (bit-exact), decode attention (per sequence and query head,
max_c |o - o_ref| <= 2e-3 * max_c |o_ref|).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from packed_cache_attention_amd import kvq

ATTN_TOL = 2e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def energy_u64(e: torch.Tensor) -> np.ndarray:
    return e.cpu().numpy().view(np.uint64)


def gpu_energy(g, xs, dev="cuda"):
    """Accumulate the block energy of each [n, H, d] tensor in xs (one call each)."""
    H, d = g.n_kv_heads, g.head_dim
    e = torch.zeros(H, d // 2, 2, dtype=torch.int64, device=dev)
    for x in xs:
        kvq.block_energy(g, x.to(dev), e)
    return e


def run_batch(seqs, k_budget, v_bits, capacity, pairing=0, kernel=kvq.DECODE_AUTO, tiles=0, scale=None,
              check_attn=True, oracle_attn=True):
    """seqs: list of (K [n, H, d] fp16, V [n, H, d] fp16, q [H_q, d] fp16) CPU tensors.

    Returns a dict of GPU and oracle results; asserts bit-exact stages."""
    dev = "cuda"
    H, d = seqs[0][0].shape[1], seqs[0][0].shape[2]
    n_q = seqs[0][2].shape[0]
    g = kvq.geom(H, k_budget, v_bits, capacity, rope_pairing=pairing)
    ogeom = oracle.Geometry(H, k_budget, v_bits, capacity, pairing=pairing)
    nseq = len(seqs)
    # ---- energies (summed over all sequences' tokens) ----
    eK = gpu_energy(g, [s[0] for s in seqs])
    eV = gpu_energy(g, [s[1] for s in seqs])
    oK = np.zeros((H, d // 2, 2), np.uint64)
    oV = np.zeros((H, d // 2, 2), np.uint64)
    for K, V, _ in seqs:
        oracle.block_energy(K.numpy(), pairing, oK)
        oracle.block_energy(V.numpy(), pairing, oV)
    np.testing.assert_array_equal(energy_u64(eK), oK)
    np.testing.assert_array_equal(energy_u64(eV), oV)
    # ---- allocation ----
    kbits = torch.empty(H, d // 2, dtype=torch.uint8, device=dev)
    ksig = torch.empty(H, d // 2, dtype=torch.float32, device=dev)
    vbits = torch.empty_like(kbits)
    vsig = torch.empty_like(ksig)
    kvq.allocate_bits(g, eK, k_budget, kvq.GREEDY, kbits, ksig)
    v_budget = 16 * (d // 2) if v_bits == 16 else v_bits * (d // 2)
    kvq.allocate_bits(g, eV, v_budget, kvq.UNIFORM, vbits, vsig)
    ob, osig = oracle.allocate(oK, k_budget, oracle.GREEDY)
    _, ovsig = oracle.allocate(oV, v_budget, oracle.UNIFORM)
    np.testing.assert_array_equal(kbits.cpu().numpy(), ob)
    np.testing.assert_array_equal(ksig.cpu().numpy().view(np.uint32), osig.view(np.uint32))
    np.testing.assert_array_equal(vsig.cpu().numpy().view(np.uint32), ovsig.view(np.uint32))
    # ---- quantize + pack (one call for the batch) ----
    region = kvq.cache_bytes(g)
    cache = torch.zeros(nseq * region, dtype=torch.uint8, device=dev)
    rows = torch.cat([s[0] for s in seqs], 0).to(dev)
    vrows = torch.cat([s[1] for s in seqs], 0).to(dev)
    lens = [s[0].shape[0] for s in seqs]
    row0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    first = torch.zeros(nseq, dtype=torch.int64, device=dev)
    n_new = torch.tensor(lens, dtype=torch.int32, device=dev)
    src0 = torch.tensor(row0, dtype=torch.int64, device=dev)
    off = torch.arange(nseq, dtype=torch.int64, device=dev) * region
    kvq.quantize_pack(g, rows, vrows, first, n_new, src0, max(lens) if lens else 0, kbits, ksig, vsig, cache, off)
    oc = np.zeros(nseq * region, np.uint8)
    for i, (K, V, _) in enumerate(seqs):
        oracle.quantize_pack(ogeom, oc[i * region:(i + 1) * region], K.numpy(), V.numpy(), 0, ob, osig, ovsig)
    gc = cache.cpu().numpy()
    if not np.array_equal(gc, oc):
        bad = np.nonzero(gc != oc)[0]
        raise AssertionError("packed bytes differ at %d positions, first %s (tile bytes %d)"
                             % (len(bad), bad[:8], ogeom.tile))
    res = {"g": g, "ogeom": ogeom, "cache": cache, "off": off, "kbits": kbits, "ksig": ksig, "vsig": vsig,
           "ob": ob, "osig": osig, "ovsig": ovsig, "oc": oc}
    if not check_attn:
        return res
    # ---- decode attention ----
    q = torch.stack([s[2] for s in seqs], 0).to(dev).contiguous()
    seq_len = torch.tensor(lens, dtype=torch.int32, device=dev)
    max_len = max(lens) if lens else 0
    ws = torch.empty(kvq.decode_workspace_bytes(g, n_q, nseq, max_len, kernel, tiles) // 4 + 4,
                     dtype=torch.float32, device=dev)
    out = torch.empty(nseq, n_q, d, dtype=torch.float32, device=dev)
    kvq.packed_decode_attn(g, q, cache, off, seq_len, max_len, kbits, ksig, vsig, out, ws, softmax_scale=scale,
                           kernel=kernel, tiles_per_split=tiles)
    o = out.cpu().numpy()
    res["out"] = o
    if oracle_attn:
        ref = np.stack([oracle.decode_attention(ogeom, oc[i * region:(i + 1) * region], seqs[i][2].numpy(), lens[i],
                                                ob, osig, ovsig, scale) for i in range(nseq)])
        res["ref"] = ref
        check_attention(o, ref)
    return res


def check_attention(o: np.ndarray, ref: np.ndarray, tol: float = ATTN_TOL):
    """Per (sequence, head): max_c |o - ref| <= tol * max_c |ref| (zero rows must be exactly zero)."""
    err = np.abs(o.astype(np.float64) - ref).max(-1)
    mag = np.abs(ref).max(-1)
    ok = np.where(mag > 0, err <= tol * mag, err == 0)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError("attention mismatch at %s: err %.3e vs max|ref| %.3e (worst rel %.3e)"
                             % (tuple(i), err[tuple(i)], mag[tuple(i)], (err / np.maximum(mag, 1e-30)).max()))
    return float((err / np.maximum(mag, 1e-30)).max())
