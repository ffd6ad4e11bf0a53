"""Seeded synthetic workloads shaped like the decode configurations studied for
"RoPE-Aware Bit Allocation for KV-Cache Quantization" (abstract: Llama-3.1-8B-,
Qwen2.5-3B- and DeepSeek-R1-Distill-Qwen-7B-shaped caches, 32K..512K contexts).

This module only draws inputs: keys, values and queries as a RoPE model would
cache them.  It holds none of the method's arithmetic and imports neither the
HIP library nor the oracle, so both sides can take their inputs from it.

Recipe (per (sequence, layer, KV head) stream, torch generator seeded with
``seed * 10**7 + stream``; draw order: outlier channels, keys, values, queries):
  * pre-RoPE key coordinate c of block i has std sigma_i (profile below), with
    3 of 128 channels (2%, rounded up) scaled x10 in the "decay" profile, or 3
    whole blocks scaled x8 in the "exp" profile (blocks picked once per config);
  * keys are rotated by RoPE at their position t (fp64, half-split pairing:
    block i = coordinates (i, i + d/2), frequency theta^(-2i/d)), then rounded to
    binary16;
  * values are N(0, 1) rounded to binary16;
  * each query is N(0, 1) rounded to binary16, rotated by RoPE at the decode
    position (fp64), and rounded to binary16 again.
"""
from __future__ import annotations

import dataclasses
import math

import torch

HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    theta: float
    seq_lens: tuple          # one entry per sequence
    k_budget: int            # sum of block widths (average bits/dim * d/2)
    v_bits: int
    profile: str             # "exp" or "decay"
    head_dim: int = HEAD_DIM

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_seq(self) -> int:
        return len(self.seq_lens)

    def with_lens(self, lens) -> "Workload":
        return dataclasses.replace(self, seq_lens=tuple(int(x) for x in lens))


def c5_lengths(seed: int = 0, n: int = 16, lo: int = 4096, hi: int = 32768):
    g = torch.Generator().manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g))


WORKLOADS = {
    # single layer / head, 1K tokens, K3V3
    "c1": Workload("c1-1layer-1kv-1k-k3v3", 1, 1, 1, 1e4, (1024,), 192, 3, "exp"),
    # Llama-3.1-8B-shaped layer: 32 q heads, 8 KV heads, 32K, K2V2
    "c2": Workload("c2-llama8b-layer-32k-k2v2", 1, 32, 8, 5e5, (32768,), 128, 2, "decay"),
    # Qwen2.5-3B-shaped decode: 36 layers, 16 q heads, 2 KV heads, 128K, K3V3
    "c3": Workload("c3-qwen3b-36layer-128k-k3v3", 36, 16, 2, 1e6, (131072,), 192, 3, "decay"),
    # same shape at 512K
    "c4": Workload("c4-qwen3b-36layer-512k-k3v3", 36, 16, 2, 1e6, (524288,), 192, 3, "decay"),
    # R1-Distill-Qwen-7B-shaped batch: 28 layers, 28 q / 4 KV heads, 16 seqs 4K..32K, K3V2
    "c5": Workload("c5-r1qwen7b-28layer-16seq-4k32k-k3v2", 28, 28, 4, 1e6, c5_lengths(), 192, 2, "decay"),
}


def block_std(profile: str, d: int = HEAD_DIM) -> torch.Tensor:
    """Per-block pre-RoPE key std (fp64, [d/2])."""
    nb = d // 2
    i = torch.arange(nb, dtype=torch.float64)
    if profile == "exp":
        return torch.exp(-3.0 * i / 64.0)
    if profile == "decay":       # log-uniform from 4 down to 1e-2 across the blocks
        return 4.0 * (0.01 / 4.0) ** (i / (nb - 1))
    raise ValueError(profile)


def exp_outlier_blocks(seed: int = 0, d: int = HEAD_DIM):
    """The 3 outlier blocks of the "exp" profile (chosen once per configuration)."""
    g = torch.Generator().manual_seed(seed)
    return torch.randperm(d // 2, generator=g)[:3]


def _rope(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """Rotate [n, d] fp64 rows by RoPE at positions pos [n] (half-split pairing)."""
    d = x.shape[-1]
    nb = d // 2
    freq = theta ** (-2.0 * torch.arange(nb, dtype=torch.float64, device=x.device) / d)
    ang = pos.to(torch.float64)[:, None] * freq[None, :]
    c, s = torch.cos(ang), torch.sin(ang)
    a, b = x[:, :nb], x[:, nb:]
    return torch.cat([a * c - b * s, a * s + b * c], dim=-1)


def stream_id(wl: Workload, seq: int, layer: int, kv_head: int) -> int:
    return (seq * wl.n_layers + layer) * wl.n_kv_heads + kv_head


def gen_head(wl: Workload, seq: int, layer: int, kv_head: int, n_tok: int, pos0: int = 0,
             seed: int = 0, device="cpu", query_pos: int | None = None):
    """Keys/values [n_tok, d] (fp16) at positions pos0.., plus the group's queries
    [g, d] (fp16) at query_pos (default: pos0 + n_tok), for one stream."""
    d = wl.head_dim
    g = torch.Generator(device=device).manual_seed(seed * 10 ** 7 + stream_id(wl, seq, layer, kv_head))
    std = block_std(wl.profile, d).to(device)
    ch_std = torch.cat([std, std])
    if wl.profile == "decay":
        out_ch = torch.randperm(d, generator=g, device=device)[:3]
        ch_std = ch_std.clone()
        ch_std[out_ch] *= 10.0
    else:
        blocks = exp_outlier_blocks(seed, d).to(device)
        ch_std = ch_std.clone()
        ch_std[blocks] *= 8.0
        ch_std[blocks + d // 2] *= 8.0
    pos = torch.arange(pos0, pos0 + n_tok, device=device)
    k = torch.randn(n_tok, d, generator=g, device=device, dtype=torch.float64) * ch_std
    k = _rope(k, pos, wl.theta).to(torch.float16)
    v = torch.randn(n_tok, d, generator=g, device=device, dtype=torch.float64).to(torch.float16)
    qp = pos0 + n_tok if query_pos is None else query_pos
    q = torch.randn(wl.group, d, generator=g, device=device, dtype=torch.float64).to(torch.float16)
    q = _rope(q.to(torch.float64), torch.full((wl.group,), qp, device=device), wl.theta).to(torch.float16)
    return k, v, q


def gen_layer(wl: Workload, seq: int, layer: int, n_tok: int | None = None, seed: int = 0, device="cpu",
              pos0: int = 0):
    """One sequence's layer: K, V [n_tok, H_kv, d] and q [H_q, d] (fp16)."""
    n = wl.seq_lens[seq] if n_tok is None else n_tok
    ks, vs, qs = [], [], []
    for h in range(wl.n_kv_heads):
        k, v, q = gen_head(wl, seq, layer, h, n, pos0=pos0, seed=seed, device=device)
        ks.append(k)
        vs.append(v)
        qs.append(q)
    return torch.stack(ks, 1), torch.stack(vs, 1), torch.cat(qs, 0)


def gen_new_token(wl: Workload, seq: int, layer: int, pos: int, step: int, seed: int = 0, device="cpu"):
    """A decode step's new K/V row [H_kv, d] and query [H_q, d] at position pos."""
    ks, vs, qs = [], [], []
    for h in range(wl.n_kv_heads):
        k, v, q = gen_head(wl, seq, layer, h, 1, pos0=pos, seed=seed + 1 + step, device=device,
                           query_pos=pos)
        ks.append(k[0])
        vs.append(v[0])
        qs.append(q)
    return torch.stack(ks, 0), torch.stack(vs, 0), torch.cat(qs, 0)


def gen_chunk_queries(wl: Workload, seq: int, layer: int, pos0: int, n_tok: int, seed: int = 0, device="cpu"):
    """A prefill chunk's queries [n_tok, H_q, d] (fp16) at positions pos0 .. pos0 + n_tok - 1:
    N(0, 1) rows rotated by RoPE at their own positions, one stream per KV head's group
    (query head = KV head * group + i)."""
    d, grp = wl.head_dim, wl.group
    pos = torch.arange(pos0, pos0 + n_tok, device=device).repeat_interleave(grp)
    out = []
    for h in range(wl.n_kv_heads):
        g = torch.Generator(device=device).manual_seed(seed * 10 ** 7 + 5 * 10 ** 6 + stream_id(wl, seq, layer, h))
        q = torch.randn(n_tok * grp, d, generator=g, device=device, dtype=torch.float64)
        out.append(_rope(q, pos, wl.theta).reshape(n_tok, grp, d).to(torch.float16))
    return torch.cat(out, 1)


def rot_signs(n_kv_heads: int, seed: int = 0, layer: int = 0, d: int = HEAD_DIM, device="cpu") -> torch.Tensor:
    """The random sign diagonal of a rotated cache: uint8 [n_kv_heads, d], 1 meaning -1,
    drawn once per (layer, KV head) from a generator seeded with seed * 10**7 + 9 * 10**6 +
    layer * n_kv_heads + head (a draw, no arithmetic of the method)."""
    out = []
    for h in range(n_kv_heads):
        g = torch.Generator().manual_seed(seed * 10 ** 7 + 9 * 10 ** 6 + layer * n_kv_heads + h)
        out.append(torch.randint(0, 2, (d,), generator=g, dtype=torch.uint8))
    return torch.stack(out).to(device)


def fp16_cache_bytes(wl: Workload) -> int:
    """Bytes an fp16 K/V cache of this workload would take (all layers, all sequences)."""
    return 2 * 2 * wl.head_dim * wl.n_kv_heads * wl.n_layers * sum(wl.seq_lens)


def ceil_to(x: int, m: int) -> int:
    return int(math.ceil(x / m) * m)
