"""CPU oracle for Block-GTQ key-cache quantization and packed-cache decode attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by the
benchmark's CPU-baseline leg; never by the product package.  It shares no code,
table or generator with the HIP library (packed_cache_attention_amd/).

The arithmetic lives in kvq_oracle.c (plain C, fp64 where the reading says fp64,
built with gcc -O2 -ffp-contract=off).  This module is a thin ctypes wrapper plus
orchestration; every function names the part of the method it follows (page:
"RoPE-Aware Bit Allocation for KV-Cache Quantization", abstract).
"""
from __future__ import annotations

import ctypes as C
import functools
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
# KVQ_ORACLE_SANITIZE=1 builds and loads an AddressSanitizer + UBSan build instead (the
# process must preload the sanitizer runtimes: LD_PRELOAD="$(gcc -print-file-name=libasan.so)
# $(gcc -print-file-name=libubsan.so)" ASAN_OPTIONS=detect_leaks=0)
_SANITIZE = os.environ.get("KVQ_ORACLE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]

PAIR_HALF, PAIR_INTERLEAVED = 0, 1
GREEDY, UNIFORM = 0, 1
TILE = 64


def build(force: bool = False) -> str:
    """Compile kvq_oracle.c with gcc (no fast-math, no FP contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-ffp-contract=off", "-fno-fast-math",
             "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wno-unused-function"] + (_SAN_FLAGS if _SANITIZE else []) +
            [_SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


@functools.lru_cache(maxsize=None)
def lib() -> C.CDLL:
    build()
    L = C.CDLL(_LIB)
    P = C.c_void_p
    I32, I64, F64 = C.c_int, C.c_int64, C.c_double
    L.or_set_threads.argtypes = [I32]
    L.or_max_threads.restype = I32
    L.or_lloyd_max.argtypes = [I32, P, P, P]
    L.or_lloyd_max.restype = I32
    L.or_round_fp16.argtypes = [P, I32, P]
    L.or_h2d.argtypes = [P, I32, P]
    L.or_block_energy.argtypes = [P, I64, I64, I64, I32, I32, I32, P]
    L.or_allocate.argtypes = [P, I32, I32, I32, I32, P, P, P]
    L.or_allocate.restype = I32
    L.or_token_scale.argtypes = [P, I32]
    L.or_token_scale.restype = C.c_float
    L.or_encode.argtypes = [P, I64, I64, I32, P, P, P, P, P, P]
    L.or_tile_bytes.argtypes = [I32, I32, I32]
    L.or_tile_bytes.restype = I64
    L.or_k_order.argtypes = [I32, I32, P, P]
    L.or_k_order.restype = I32
    L.or_pack.argtypes = [P, I32, I32, I32, I32, P, I64, I64, P, P, P, P]
    L.or_unpack.argtypes = [P, I32, I32, I32, I32, P, I64, I64, P, P, P, P]
    L.or_dequant.argtypes = [P, I64, I32, P, P, P, P, P, P]
    L.or_attend.argtypes = [P, P, P, I64, I32, F64, P]
    L.or_decode_attention.argtypes = [P, I64, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, I64, F64, P]
    L.or_decode_attention_window.argtypes = [P, I64, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, I64, P, P, I64,
                                             F64, P]
    L.or_prefill_attention.argtypes = [P, I64, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, I64, I64, F64, P]
    L.or_attend_partial.argtypes = [P, P, P, I64, I32, F64, P, P, P]
    L.or_merge_partials.argtypes = [P, I64, I32, I32, P]
    L.or_hadamard_units.argtypes = [P, I32, P, P]
    L.or_hadamard_f32.argtypes = [P, I32, P, P]
    L.or_rot_encode.argtypes = [P, I64, I64, I32, I32, P, P, P, P, P]
    L.or_rot_query.argtypes = [P, I32, P, C.c_float, P]
    L.or_rot_back.argtypes = [P, I32, P, P]
    return L


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


# --------------------------------------------------------------------------
# Codebooks (TQ-MSE scalar quantizer read as Gaussian Lloyd-Max, 2^w levels)
# --------------------------------------------------------------------------

@functools.lru_cache(maxsize=None)
def codebook(w: int) -> dict:
    """Lloyd-Max codebook of N(0,1) with 2^w levels, solved in kvq_oracle.c.

    Returns exact levels (fp64), their binary16 patterns and values, the binary32
    midpoint thresholds (index 0 unused), the ideal distortion D and the
    fixed-point residual.
    """
    n = 1 << w
    cent = np.zeros(n, np.float64)
    D = np.zeros(1, np.float64)
    res = np.zeros(1, np.float64)
    steps = lib().or_lloyd_max(w, _p(cent), _p(D), _p(res))
    if steps < 0:
        raise RuntimeError("Lloyd-Max solve failed")
    h16 = np.zeros(n, np.uint16)
    lib().or_round_fp16(_p(cent), n, _p(h16))
    lv = np.zeros(n, np.float64)
    lib().or_h2d(_p(h16), n, _p(lv))
    thr = np.zeros(n, np.float32)
    lv32 = lv.astype(np.float32)
    for j in range(1, n):
        s = np.float32(lv32[j - 1] + lv32[j])
        thr[j] = np.float32(s * np.float32(0.5))
        # the midpoint of two neighbouring binary16 levels is exact in binary32
        assert float(thr[j]) == 0.5 * (float(lv[j - 1]) + float(lv[j]))
    return {"levels": cent, "levels_fp16": h16, "levels_h": lv, "thresholds": thr,
            "D": float(D[0]), "resid": float(res[0]), "newton_steps": steps}


@functools.lru_cache(maxsize=None)
def tables() -> dict:
    """Concatenated per-width tables plus the binary32 distortion drops dD[b], b=0..7."""
    thr_off = np.zeros(17, np.int32)
    lev_off = np.zeros(17, np.int32)
    thr, lev = [], []
    off = 0
    for w in range(1, 9):
        cb = codebook(w)
        thr_off[w] = off
        lev_off[w] = off
        thr.append(cb["thresholds"])
        lev.append(cb["levels_fp16"])
        off += 1 << w
    D = [1.0] + [codebook(w)["D"] for w in range(1, 9)]
    dD = np.array([D[b] - D[b + 1] for b in range(8)], np.float64)
    return {"thr": np.concatenate(thr).astype(np.float32), "thr_off": thr_off,
            "lev": np.concatenate(lev).astype(np.uint16), "lev_off": lev_off,
            "D": np.array(D), "dD64": dD, "dD": dD.astype(np.float32)}


# --------------------------------------------------------------------------
# Energy and allocation
# --------------------------------------------------------------------------

def block_energy(x16: np.ndarray, pairing: int = PAIR_HALF, energy: np.ndarray | None = None) -> np.ndarray:
    """Exact per-block energy, sum over tokens of the block's squared norm.

    x16: binary16 patterns (uint16) or float16, shape [n_tok, n_heads, d].
    Returns (or accumulates into) uint64 [n_heads, d/2, 2] (low, high limbs of a
    128-bit count of 2^-48 units).
    """
    x = np.ascontiguousarray(x16).view(np.uint16)
    n, H, d = x.shape
    if energy is None:
        energy = np.zeros((H, d // 2, 2), np.uint64)
    lib().or_block_energy(_p(x), n, H * d, d, H, d, pairing, _p(energy))
    return energy


def energy_to_int(energy: np.ndarray) -> np.ndarray:
    """uint64 limb pairs -> Python ints (object array)."""
    lo = energy[..., 0].astype(object)
    hi = energy[..., 1].astype(object)
    return lo + (hi << 64)


def allocate(energy: np.ndarray, budget: int, mode: int = GREEDY):
    """Greedy (or uniform) integer widths and per-block scales; see or_allocate."""
    e = np.ascontiguousarray(energy, dtype=np.uint64)
    nu, nb = e.shape[0], e.shape[1]
    bits = np.zeros((nu, nb), np.uint8)
    sig = np.zeros((nu, nb), np.float32)
    dD = tables()["dD"]
    rc = lib().or_allocate(_p(e), nu, nb, budget, mode, _p(dD), _p(bits), _p(sig))
    if rc != 0:
        raise ValueError("invalid budget %d for %d blocks (mode %d)" % (budget, nb, mode))
    return bits, sig


# --------------------------------------------------------------------------
# Quantization, layout, attention
# --------------------------------------------------------------------------

def coord_map(d: int, pairing: int):
    """(p, q) coordinate arrays of the d/2 blocks."""
    i = np.arange(d // 2)
    if pairing == PAIR_HALF:
        return i, i + d // 2
    return 2 * i, 2 * i + 1


def per_coord(block_vals: np.ndarray, d: int, pairing: int) -> np.ndarray:
    p, q = coord_map(d, pairing)
    out = np.zeros(d, block_vals.dtype)
    out[p] = block_vals
    out[q] = block_vals
    return out


def token_scale(x16: np.ndarray) -> float:
    x = np.ascontiguousarray(x16).view(np.uint16)
    return float(lib().or_token_scale(_p(x), x.shape[-1]))


def encode(x16: np.ndarray, width_c: np.ndarray, sig_c: np.ndarray):
    """Codes [n, d] (uint16) and per-token scales [n] for one head's tokens [n, d]."""
    x = np.ascontiguousarray(x16).view(np.uint16)
    n, d = x.shape
    T = tables()
    codes = np.zeros((n, d), np.uint16)
    scale = np.zeros(n, np.float32)
    w = np.ascontiguousarray(width_c, np.int32)
    s = np.ascontiguousarray(sig_c, np.float32)
    lib().or_encode(_p(x), n, d, d, _p(w), _p(s), _p(T["thr"]), _p(T["thr_off"]), _p(codes), _p(scale))
    return codes, scale


def tile_bytes(d: int, k_budget: int, v_bits: int) -> int:
    return int(lib().or_tile_bytes(d, k_budget, v_bits))


def k_order(bits_blk: np.ndarray, d: int, pairing: int) -> np.ndarray:
    b = np.ascontiguousarray(bits_blk, np.uint8)
    order = np.zeros(2 * len(b), np.int32)
    n = lib().or_k_order(d, pairing, _p(b), _p(order))
    return order[:n]


def pack(region: np.ndarray, d, pairing, k_budget, v_bits, kbits_blk, first_slot, kcodes, vcodes, kscale, vscale):
    """OR one head's tokens into its (zero-initialised) tile sequence `region` (uint8)."""
    kb = np.ascontiguousarray(kbits_blk, np.uint8)
    n = kcodes.shape[0]
    lib().or_pack(_p(region), d, pairing, k_budget, v_bits, _p(kb), first_slot, n,
                  _p(np.ascontiguousarray(kcodes, np.uint16)), _p(np.ascontiguousarray(vcodes, np.uint16)),
                  _p(np.ascontiguousarray(kscale, np.float32)), _p(np.ascontiguousarray(vscale, np.float32)))


def unpack(region: np.ndarray, d, pairing, k_budget, v_bits, kbits_blk, first_slot, n):
    kb = np.ascontiguousarray(kbits_blk, np.uint8)
    kc = np.zeros((n, d), np.uint16)
    vc = np.zeros((n, d), np.uint16)
    ks = np.zeros(n, np.float32)
    vs = np.zeros(n, np.float32)
    lib().or_unpack(_p(np.ascontiguousarray(region)), d, pairing, k_budget, v_bits, _p(kb), first_slot, n,
                    _p(kc), _p(vc), _p(ks), _p(vs))
    return kc, vc, ks, vs


def dequant(codes: np.ndarray, width_c: np.ndarray, sig_c: np.ndarray, scale: np.ndarray) -> np.ndarray:
    T = tables()
    n, d = codes.shape
    out = np.zeros((n, d), np.float64)
    lib().or_dequant(_p(np.ascontiguousarray(codes, np.uint16)), n, d, _p(np.ascontiguousarray(width_c, np.int32)),
                     _p(np.ascontiguousarray(sig_c, np.float32)), _p(np.ascontiguousarray(scale, np.float32)),
                     _p(T["lev"]), _p(T["lev_off"]), _p(out))
    return out


def attend(q: np.ndarray, khat: np.ndarray, vhat: np.ndarray, scale: float) -> np.ndarray:
    n, d = khat.shape
    o = np.zeros(d, np.float64)
    lib().or_attend(_p(np.ascontiguousarray(q, np.float64)), _p(np.ascontiguousarray(khat, np.float64)),
                    _p(np.ascontiguousarray(vhat, np.float64)), n, d, scale, _p(o))
    return o


def attend_partial(q: np.ndarray, khat: np.ndarray, vhat: np.ndarray, scale: float):
    """Partial (m, l, o) of one query over a chunk of tokens (m in log2 units, o
    unnormalised) -- the split-K format; see or_attend_partial."""
    n, d = khat.shape
    o = np.zeros(d, np.float64)
    m = C.c_double()
    l_ = C.c_double()
    lib().or_attend_partial(_p(np.ascontiguousarray(q, np.float64)), _p(np.ascontiguousarray(khat, np.float64)),
                            _p(np.ascontiguousarray(vhat, np.float64)), n, d, scale, C.byref(m), C.byref(l_), _p(o))
    return m.value, l_.value, o


def merge_partials(partials: np.ndarray) -> np.ndarray:
    """fp64 log-sum-exp merge of partials [rows, n_split, d + 2] (binary32: m, l, o)."""
    p = np.ascontiguousarray(partials, np.float32)
    rows, ns, d2 = p.shape
    out = np.zeros((rows, d2 - 2), np.float64)
    lib().or_merge_partials(_p(p), rows, ns, d2 - 2, _p(out))
    return out


class Geometry:
    """Shape of one layer's packed cache (mirrors the library's geometry struct)."""

    def __init__(self, n_kv_heads, k_budget, v_bits, capacity_tokens, head_dim=128, pairing=PAIR_HALF):
        assert capacity_tokens % TILE == 0
        self.d, self.H, self.kb, self.vb = head_dim, n_kv_heads, k_budget, v_bits
        self.capacity, self.pairing = capacity_tokens, pairing
        self.n_tiles = capacity_tokens // TILE
        self.tile = tile_bytes(head_dim, k_budget, v_bits)
        self.seq_bytes = self.H * self.n_tiles * self.tile


def quantize_pack(geom: Geometry, region: np.ndarray, k16: np.ndarray, v16: np.ndarray, first_slot: int,
                  kbits: np.ndarray, ksig: np.ndarray, vsig: np.ndarray):
    """Quantize tokens k16/v16 [n, H, d] of one sequence into `region` at first_slot.

    Returns per-head (kcodes, vcodes, kscale, vscale) for separate comparison.
    """
    d, H = geom.d, geom.H
    out = []
    vw = np.full(d, geom.vb, np.int32)
    for h in range(H):
        kw = per_coord(kbits[h].astype(np.int32), d, geom.pairing)
        kc, ks = encode(np.ascontiguousarray(k16[:, h, :]), kw, per_coord(ksig[h], d, geom.pairing))
        vc, vs = encode(np.ascontiguousarray(v16[:, h, :]), vw, per_coord(vsig[h], d, geom.pairing))
        view = region[h * geom.n_tiles * geom.tile:(h + 1) * geom.n_tiles * geom.tile]
        pack(view, d, geom.pairing, geom.kb, geom.vb, kbits[h], first_slot, kc, vc, ks, vs)
        out.append((kc, vc, ks, vs))
    return out


def decode_attention(geom: Geometry, region: np.ndarray, q16: np.ndarray, seq_len: int,
                     kbits: np.ndarray, ksig: np.ndarray, vsig: np.ndarray, scale: float | None = None) -> np.ndarray:
    """Exact fp64 attention of q16 [H_q, d] over slots [0, seq_len) of one sequence's region."""
    T = tables()
    d = geom.d
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nq = q16.shape[0]
    out = np.zeros((nq, d), np.float64)
    lib().or_decode_attention(_p(np.ascontiguousarray(region)), geom.n_tiles, geom.H, nq, d, geom.pairing,
                              geom.kb, geom.vb, _p(np.ascontiguousarray(kbits, np.uint8)),
                              _p(np.ascontiguousarray(ksig, np.float32)), _p(np.ascontiguousarray(vsig, np.float32)),
                              _p(T["lev"]), _p(T["lev_off"]), _p(np.ascontiguousarray(q16).view(np.uint16)),
                              seq_len, float(scale), _p(out))
    return out


def decode_attention_window(geom: Geometry, region: np.ndarray, q16: np.ndarray, n_packed: int,
                            wk16: np.ndarray, wv16: np.ndarray, kbits: np.ndarray, ksig: np.ndarray,
                            vsig: np.ndarray, scale: float | None = None) -> np.ndarray:
    """Exact fp64 attention of q16 [H_q, d] over packed slots [0, n_packed) followed by
    the window tokens wk16/wv16 [n_win, H, d] (binary16, sequence order) taken exactly
    -- the fp16 recent-window variant (the most recent tokens kept unquantized)."""
    T = tables()
    d = geom.d
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nq = q16.shape[0]
    wk = np.ascontiguousarray(wk16).view(np.uint16).reshape(-1, geom.H, d)
    wv = np.ascontiguousarray(wv16).view(np.uint16).reshape(-1, geom.H, d)
    assert wk.shape == wv.shape
    out = np.zeros((nq, d), np.float64)
    lib().or_decode_attention_window(
        _p(np.ascontiguousarray(region)), geom.n_tiles, geom.H, nq, d, geom.pairing, geom.kb, geom.vb,
        _p(np.ascontiguousarray(kbits, np.uint8)), _p(np.ascontiguousarray(ksig, np.float32)),
        _p(np.ascontiguousarray(vsig, np.float32)), _p(T["lev"]), _p(T["lev_off"]),
        _p(np.ascontiguousarray(q16).view(np.uint16)), n_packed, _p(wk), _p(wv), wk.shape[0], float(scale), _p(out))
    return out


def prefill_attention(geom: Geometry, region: np.ndarray, q16: np.ndarray, q_start: int,
                      kbits: np.ndarray, ksig: np.ndarray, vsig: np.ndarray, scale: float | None = None) -> np.ndarray:
    """Causal fp64 attention of a chunk of queries q16 [n_tok, H_q, d] whose first sits
    at position q_start: query j attends packed slots [0, q_start + j] (its own token
    included, so the chunk must already be packed).  Row j equals decode attention at
    length q_start + j + 1."""
    T = tables()
    d = geom.d
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qq = np.ascontiguousarray(q16).view(np.uint16)
    n_tok, nq = qq.shape[0], qq.shape[1]
    assert q_start + n_tok <= geom.capacity
    out = np.zeros((n_tok, nq, d), np.float64)
    lib().or_prefill_attention(_p(np.ascontiguousarray(region)), geom.n_tiles, geom.H, nq, d, geom.pairing,
                               geom.kb, geom.vb, _p(np.ascontiguousarray(kbits, np.uint8)),
                               _p(np.ascontiguousarray(ksig, np.float32)),
                               _p(np.ascontiguousarray(vsig, np.float32)), _p(T["lev"]), _p(T["lev_off"]),
                               _p(qq), int(q_start), n_tok, float(scale), _p(out))
    return out


# --------------------------------------------------------------------------
# TQ-MSE proper: randomized Walsh-Hadamard rotation (next-3 variant)
# --------------------------------------------------------------------------

def rot_sigma() -> np.float32:
    """The rotated codebook's coordinate scale 1/sqrt(128) = sqrt(2)/16 rounded to
    binary32 (sqrt(2) correctly rounded in fp64, then to binary32, then an exact /16)."""
    return np.float32(np.float32(np.sqrt(2.0)) / np.float32(16.0))


def hadamard_units(x16: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Exact S_i = sum_j H[i][j] sg_j x_j of one binary16 row, as int64 counts of 2^-24."""
    x = np.ascontiguousarray(x16).view(np.uint16)
    out = np.zeros(x.shape[-1], np.int64)
    lib().or_hadamard_units(_p(x), x.shape[-1], _p(np.ascontiguousarray(signs, np.uint8)), _p(out))
    return out


def hadamard_f32(x16: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """RN32 of the exact rotated sums of one binary16 row."""
    x = np.ascontiguousarray(x16).view(np.uint16)
    out = np.zeros(x.shape[-1], np.float32)
    lib().or_hadamard_f32(_p(x), x.shape[-1], _p(np.ascontiguousarray(signs, np.uint8)), _p(out))
    return out


def rot_encode(x16: np.ndarray, w: int, signs: np.ndarray):
    """Codes [n, d] and per-token scales [n] of binary16 rows [n, d] under the rotation,
    every coordinate at width w (1..8); see or_rot_encode."""
    x = np.ascontiguousarray(x16).view(np.uint16)
    n, d = x.shape
    T = tables()
    codes = np.zeros((n, d), np.uint16)
    scale = np.zeros(n, np.float32)
    lib().or_rot_encode(_p(x), n, d, d, w, _p(np.ascontiguousarray(signs, np.uint8)), _p(T["thr"]),
                        _p(T["thr_off"]), _p(codes), _p(scale))
    return codes, scale


def rot_query(q16: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """A binary16 query rotated once: RN16(RN32(RN32(S_i) * rot_sigma()))."""
    q = np.ascontiguousarray(q16).view(np.uint16)
    out = np.zeros(q.shape[-1], np.uint16)
    lib().or_rot_query(_p(q), q.shape[-1], _p(np.ascontiguousarray(signs, np.uint8)), float(rot_sigma()), _p(out))
    return out


def rot_back(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """R^T y = diag(sg) H y / sqrt(d) in fp64 (an output rotated back)."""
    yy = np.ascontiguousarray(y, np.float64)
    out = np.zeros(yy.shape[-1], np.float64)
    lib().or_rot_back(_p(yy), yy.shape[-1], _p(np.ascontiguousarray(signs, np.uint8)), _p(out))
    return out


def quantize_pack_rot(geom: "Geometry", region: np.ndarray, k16: np.ndarray, v16: np.ndarray, first_slot: int,
                      k_signs: np.ndarray, v_signs: np.ndarray | None, vsig: np.ndarray | None):
    """The rotated variant of quantize_pack: keys rotated and coded at the uniform width
    k_budget / (d/2) (no allocation: rotation spreads every block's energy over all
    coordinates); values rotated the same way when v_signs is given, else coded as in
    quantize_pack with the per-block scales vsig.  Packed in layout v1 with uniform
    key widths.  Returns per-head (kcodes, vcodes, kscale, vscale)."""
    d, H = geom.d, geom.H
    nb = d // 2
    assert geom.kb % nb == 0 and 1 <= geom.kb // nb <= 8 and geom.vb <= 8
    wk = geom.kb // nb
    kbits = np.full((H, nb), wk, np.uint8)
    vw = np.full(d, geom.vb, np.int32)
    out = []
    for h in range(H):
        kc, ks = rot_encode(np.ascontiguousarray(k16[:, h, :]), wk, k_signs[h])
        if v_signs is not None:
            vc, vs = rot_encode(np.ascontiguousarray(v16[:, h, :]), geom.vb, v_signs[h])
        else:
            vc, vs = encode(np.ascontiguousarray(v16[:, h, :]), vw, per_coord(vsig[h], d, geom.pairing))
        view = region[h * geom.n_tiles * geom.tile:(h + 1) * geom.n_tiles * geom.tile]
        pack(view, d, geom.pairing, geom.kb, geom.vb, kbits[h], first_slot, kc, vc, ks, vs)
        out.append((kc, vc, ks, vs))
    return out


def decode_attention_rot(geom: "Geometry", region: np.ndarray, q16: np.ndarray, seq_len: int, k_signs: np.ndarray,
                         v_signs: np.ndarray | None, vsig: np.ndarray | None,
                         scale: float | None = None) -> np.ndarray:
    """Exact fp64 attention of the rotated variant for one sequence: each query head is
    rotated once (rot_query with its KV head's key signs), the keys are dequantized in
    rotated coordinates (s * rot_sigma() * level), softmax attention as usual, and with
    rotated values the output is rotated back once (rot_back with the value signs)."""
    d, H = geom.d, geom.H
    nb = d // 2
    wk = geom.kb // nb
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nq = q16.shape[0]
    g = nq // H
    sig_r = np.full(d, rot_sigma(), np.float32)
    out = np.zeros((nq, d), np.float64)
    kbits = np.full(nb, wk, np.uint8)
    for kv in range(H):
        view = region[kv * geom.n_tiles * geom.tile:(kv + 1) * geom.n_tiles * geom.tile]
        kc, vc, ks, vs = unpack(view, d, geom.pairing, geom.kb, geom.vb, kbits, 0, seq_len)
        khat = dequant(kc, np.full(d, wk, np.int32), sig_r, ks)
        vsig_c = sig_r if v_signs is not None else per_coord(vsig[kv], d, geom.pairing)
        vhat = dequant(vc, np.full(d, geom.vb, np.int32), vsig_c, vs)
        for h in range(kv * g, (kv + 1) * g):
            qr = rot_query(q16[h], k_signs[kv]).view(np.float16).astype(np.float64)
            o = attend(qr, khat, vhat, scale)
            out[h] = rot_back(o, v_signs[kv]) if v_signs is not None else o
    return out


def set_threads(n: int) -> int:
    """Thread count of the oracle's OpenMP loops (timing only; results do not depend on
    it).  Returns the count now in force."""
    lib().or_set_threads(int(n))
    return int(lib().or_max_threads())
