"""ctypes binding of libkvq.so (C ABI in include/kvq.h).

Argument marshalling only: torch tensors become raw device pointers and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  Nothing here falls back to a CPU path: if the library has not been
built, or a call is rejected, an exception is raised.
"""
from __future__ import annotations

import ctypes as C
import functools
import os

import torch  # noqa: F401  (load torch's HIP runtime before the library maps its own soname)

# KVQ_LIBRARY names another build of the same library (e.g. the host-sanitized one)
_LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

OK = 0
PAIR_HALF, PAIR_INTERLEAVED = 0, 1
GREEDY, UNIFORM = 0, 1
DECODE_AUTO, DECODE_GENERIC, DECODE_MFMA = 0, 1, 2
LAYOUT_VERSION = 1
TILE = 64


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))
        self.status = status


class Geom(C.Structure):
    _fields_ = [("layout_version", C.c_int32), ("head_dim", C.c_int32), ("n_kv_heads", C.c_int32),
                ("rope_pairing", C.c_int32), ("k_budget", C.c_int32), ("v_bits", C.c_int32),
                ("capacity_tokens", C.c_int64)]


def geom(n_kv_heads: int, k_budget: int, v_bits: int, capacity_tokens: int, head_dim: int = 128,
         rope_pairing: int = PAIR_HALF) -> Geom:
    return Geom(LAYOUT_VERSION, head_dim, n_kv_heads, rope_pairing, k_budget, v_bits, capacity_tokens)


@functools.lru_cache(maxsize=None)
def lib() -> C.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libkvq.so is not built (run __graft_entry__.build() or "
                           "packed_cache_attention_amd/csrc/build.py)")
    L = C.CDLL(_LIB_PATH)
    P, G = C.c_void_p, C.POINTER(Geom)
    I32, I64, F32, SZ = C.c_int32, C.c_int64, C.c_float, C.c_size_t
    L.kvq_version.restype = I32
    L.kvq_status_string.argtypes = [I32]
    L.kvq_status_string.restype = C.c_char_p
    L.kvq_tile_bytes.argtypes = [G]
    L.kvq_tile_bytes.restype = I64
    L.kvq_cache_bytes.argtypes = [G]
    L.kvq_cache_bytes.restype = I64
    L.kvq_get_codebook.argtypes = [I32, P, P, P]
    L.kvq_get_codebook.restype = I32
    L.kvq_block_energy.argtypes = [G, P, I64, I64, I64, P, P]
    L.kvq_block_energy.restype = I32
    L.kvq_allocate_bits.argtypes = [G, P, I32, I32, I32, P, P, P]
    L.kvq_allocate_bits.restype = I32
    L.kvq_quantize_pack.argtypes = [G, P, P, I64, I64, I32, P, P, P, I32, P, P, P, P, P, P]
    L.kvq_quantize_pack.restype = I32
    L.kvq_decode_workspace_bytes.argtypes = [G, I32, I32, I64]
    L.kvq_decode_workspace_bytes.restype = I64
    L.kvq_decode_workspace_bytes_ex.argtypes = [G, I32, I32, I64, I32, I32]
    L.kvq_decode_workspace_bytes_ex.restype = I64
    L.kvq_packed_decode_attn.argtypes = [G, I32, P, P, P, P, I32, I64, P, P, P, F32, P, P, SZ, P]
    L.kvq_packed_decode_attn.restype = I32
    L.kvq_packed_decode_attn_ex.argtypes = [G, I32, P, P, P, P, I32, I64, P, P, P, F32, P, P, SZ, I32, I32, P]
    L.kvq_packed_decode_attn_ex.restype = I32
    L.kvq_packed_decode_attn_noalloc.argtypes = [G, I32, P, P, P, P, I32, I64, P, P, P, F32, P, P]
    L.kvq_packed_decode_attn_noalloc.restype = I32
    L.kvq_decode_partials.argtypes = [G, I32, P, P, P, P, I32, I64, P, P, P, F32, P, SZ, I32, I32, P]
    L.kvq_decode_partials.restype = I32
    L.kvq_merge_partials.argtypes = [I32, I32, I32, P, P, P]
    L.kvq_merge_partials.restype = I32
    L.kvq_decode_n_split.argtypes = [G, I32, I32, I64, I32, I32]
    L.kvq_decode_n_split.restype = I32
    L.kvq_decode_step_partials.argtypes = [G, I32, P, P, P, I64, I64, P, P, P, I32, I64, P, P, P, F32, P, SZ, I32,
                                           I32, P]
    L.kvq_decode_step_partials.restype = I32
    L.kvq_decode_step.argtypes = [G, I32, P, P, P, I64, I64, P, P, P, I32, I64, P, P, P, F32, P, P, SZ, I32, I32, P]
    L.kvq_decode_step.restype = I32
    L.kvq_window_workspace_bytes.argtypes = [G, I32, I32, I32, I64, I32, I32]
    L.kvq_window_workspace_bytes.restype = I64
    L.kvq_window_decode_attn.argtypes = [G, I32, I32, P, P, P, P, P, P, I32, I64, P, P, P, F32, P, P, SZ, I32, I32,
                                         P]
    L.kvq_window_decode_attn.restype = I32
    L.kvq_window_decode_step.argtypes = [G, I32, I32, P, P, P, I64, I64, P, P, P, P, P, I32, I64, P, P, P, F32, P, P,
                                         SZ, I32, I32, P]
    L.kvq_window_decode_step.restype = I32
    L.kvq_decode_plan.argtypes = [G, I32, I32, I64, I32, I32, P, P, P, P]
    L.kvq_decode_plan.restype = I32
    L.kvq_prefill_plan.argtypes = [G, I32, I32, I32, I64, I32, P, P]
    L.kvq_prefill_plan.restype = I32
    L.kvq_prefill_workspace_bytes.argtypes = [G, I32, I32, I32, I64, I32]
    L.kvq_prefill_workspace_bytes.restype = I64
    L.kvq_packed_prefill_attn.argtypes = [G, I32, P, P, P, P, P, I32, I32, I64, P, P, P, F32, P, P, SZ, I32, P]
    L.kvq_packed_prefill_attn.restype = I32
    L.kvq_rot_quantize_pack.argtypes = [G, P, P, I64, I64, I32, P, P, P, I32, P, P, P, P, P, P]
    L.kvq_rot_quantize_pack.restype = I32
    L.kvq_rot_queries.argtypes = [G, I32, I32, P, P, P, P]
    L.kvq_rot_queries.restype = I32
    L.kvq_rot_back.argtypes = [G, I32, I32, P, P, P]
    L.kvq_rot_back.restype = I32
    L.kvq_rot_decode_prepare.argtypes = [G, I32, I32, P, P, P, P, I64, I64, P, P, P, P, P, P, P]
    L.kvq_rot_decode_prepare.restype = I32
    L.kvq_rot_decode_step_partials.argtypes = [G, I32, P, P, P, I64, I64, P, P, P, I32, I64, P, P, P, P, P, F32, P,
                                               SZ, I32, P]
    L.kvq_rot_decode_step_partials.restype = I32
    L.kvq_read_probe.argtypes = [P, I64, P, I32, P]
    L.kvq_read_probe.restype = I32
    if L.kvq_version() != LAYOUT_VERSION:
        raise RuntimeError("libkvq.so layout version mismatch")
    return L


EXPORTS = ["kvq_version", "kvq_status_string", "kvq_tile_bytes", "kvq_cache_bytes", "kvq_get_codebook",
           "kvq_block_energy", "kvq_allocate_bits", "kvq_quantize_pack", "kvq_decode_workspace_bytes",
           "kvq_decode_workspace_bytes_ex", "kvq_packed_decode_attn", "kvq_packed_decode_attn_ex",
           "kvq_packed_decode_attn_noalloc",
           "kvq_decode_partials", "kvq_merge_partials", "kvq_decode_n_split", "kvq_decode_plan",
           "kvq_decode_step_partials", "kvq_decode_step", "kvq_window_decode_attn", "kvq_window_decode_step",
           "kvq_window_workspace_bytes", "kvq_prefill_plan", "kvq_prefill_workspace_bytes",
           "kvq_packed_prefill_attn", "kvq_read_probe", "kvq_rot_quantize_pack", "kvq_rot_queries", "kvq_rot_back",
           "kvq_rot_decode_prepare", "kvq_rot_decode_step_partials"]


def status_string(st: int) -> str:
    return lib().kvq_status_string(st).decode()


def _check(fn: str, st: int):
    if st != OK:
        raise KvqError(fn, st)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    return stream if isinstance(stream, int) else stream.cuda_stream


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)


# ---------------------------------------------------------------- host-only queries

def tile_bytes(g: Geom) -> int:
    r = lib().kvq_tile_bytes(C.byref(g))
    if r < 0:
        raise KvqError("kvq_tile_bytes", r)
    return r


def cache_bytes(g: Geom) -> int:
    r = lib().kvq_cache_bytes(C.byref(g))
    if r < 0:
        raise KvqError("kvq_cache_bytes", r)
    return r


def decode_workspace_bytes(g: Geom, n_q_heads: int, n_seq: int, max_len: int, kernel: int = DECODE_AUTO,
                           tiles_per_split: int = 0) -> int:
    r = lib().kvq_decode_workspace_bytes_ex(C.byref(g), n_q_heads, n_seq, max_len, kernel, tiles_per_split)
    if r < 0:
        raise KvqError("kvq_decode_workspace_bytes", r)
    return r


def get_codebook(w: int):
    import numpy as np
    lev = np.zeros(1 << w, np.uint16)
    thr = np.zeros(1 << w, np.float32)
    dd = np.zeros(8, np.float32)
    _check("kvq_get_codebook", lib().kvq_get_codebook(w, lev.ctypes.data, thr.ctypes.data, dd.ctypes.data))
    return lev, thr, dd


# ---------------------------------------------------------------- device calls

def block_energy(g: Geom, x: torch.Tensor, energy: torch.Tensor, stream=None):
    """Accumulate exact block energies of x [n_tok, n_kv, d] (fp16, d contiguous) into
    energy [n_kv, d/2, 2] (int64 storage of uint64 limbs)."""
    _dev(x, "x")
    _dev(energy, "energy")
    assert x.dtype == torch.float16 and x.dim() == 3 and x.stride(2) == 1
    assert energy.dtype == torch.int64 and energy.is_contiguous()
    _check("kvq_block_energy", lib().kvq_block_energy(C.byref(g), _ptr(x), x.shape[0], x.stride(0), x.stride(1),
                                                       _ptr(energy), _stream(stream)))


def allocate_bits(g: Geom, energy: torch.Tensor, budget: int, mode: int, bits: torch.Tensor, sigma: torch.Tensor,
                  stream=None):
    for t, n in ((energy, "energy"), (bits, "bits"), (sigma, "sigma")):
        _dev(t, n)
    assert bits.dtype == torch.uint8 and sigma.dtype == torch.float32 and energy.dtype == torch.int64
    n_units = energy.shape[0]
    _check("kvq_allocate_bits", lib().kvq_allocate_bits(C.byref(g), _ptr(energy), n_units, budget, mode,
                                                         _ptr(bits), _ptr(sigma), _stream(stream)))


def quantize_pack(g: Geom, k: torch.Tensor, v: torch.Tensor, first_slot: torch.Tensor, n_new: torch.Tensor,
                  src_row0: torch.Tensor, max_new: int, k_bits: torch.Tensor, k_sigma: torch.Tensor,
                  v_sigma: torch.Tensor, cache: torch.Tensor, seq_byte_off: torch.Tensor, stream=None):
    """k, v: [rows, n_kv, d] fp16 with identical strides; metadata int64/int32 device vectors."""
    assert k.dtype == torch.float16 and v.dtype == torch.float16 and k.stride() == v.stride() and k.stride(2) == 1
    assert first_slot.dtype == torch.int64 and src_row0.dtype == torch.int64 and seq_byte_off.dtype == torch.int64
    assert n_new.dtype == torch.int32 and cache.dtype == torch.uint8
    n_seq = first_slot.shape[0]
    _check("kvq_quantize_pack", lib().kvq_quantize_pack(
        C.byref(g), _ptr(k), _ptr(v), k.stride(0), k.stride(1), n_seq, _ptr(first_slot), _ptr(n_new),
        _ptr(src_row0), max_new, _ptr(k_bits), _ptr(k_sigma), _ptr(v_sigma), _ptr(cache), _ptr(seq_byte_off),
        _stream(stream)))


def packed_decode_attn(g: Geom, q: torch.Tensor, cache: torch.Tensor, seq_byte_off: torch.Tensor,
                       seq_len: torch.Tensor, max_len: int, k_bits: torch.Tensor, k_sigma: torch.Tensor,
                       v_sigma: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                       softmax_scale: float | None = None, kernel: int = DECODE_AUTO, tiles_per_split: int = 0,
                       stream=None):
    """q [n_seq, n_q, 128] fp16 contiguous -> out [n_seq, n_q, 128] fp32."""
    assert q.dtype == torch.float16 and q.is_contiguous() and out.dtype == torch.float32 and out.is_contiguous()
    assert seq_len.dtype == torch.int32 and seq_byte_off.dtype == torch.int64
    n_seq, n_q = q.shape[0], q.shape[1]
    if softmax_scale is None:
        softmax_scale = g.head_dim ** -0.5
    _check("kvq_packed_decode_attn", lib().kvq_packed_decode_attn_ex(
        C.byref(g), n_q, _ptr(q), _ptr(cache), _ptr(seq_byte_off), _ptr(seq_len), n_seq, max_len, _ptr(k_bits),
        _ptr(k_sigma), _ptr(v_sigma), float(softmax_scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), kernel, tiles_per_split, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 8 << 20  # KVQ_NOALLOC_SCRATCH_BYTES


def packed_decode_attn_noalloc(g: Geom, q: torch.Tensor, cache: torch.Tensor, seq_byte_off: torch.Tensor,
                               seq_len: torch.Tensor, max_len: int, k_bits: torch.Tensor, k_sigma: torch.Tensor,
                               v_sigma: torch.Tensor, out: torch.Tensor, softmax_scale: float | None = None,
                               stream=None):
    """As packed_decode_attn (automatic plan) with the partials in the library's own
    device array instead of a workspace: nothing is allocated."""
    assert q.dtype == torch.float16 and q.is_contiguous() and out.dtype == torch.float32 and out.is_contiguous()
    assert seq_len.dtype == torch.int32 and seq_byte_off.dtype == torch.int64
    n_seq, n_q = q.shape[0], q.shape[1]
    if softmax_scale is None:
        softmax_scale = g.head_dim ** -0.5
    _check("kvq_packed_decode_attn_noalloc", lib().kvq_packed_decode_attn_noalloc(
        C.byref(g), n_q, _ptr(q), _ptr(cache), _ptr(seq_byte_off), _ptr(seq_len), n_seq, max_len, _ptr(k_bits),
        _ptr(k_sigma), _ptr(v_sigma), float(softmax_scale), _ptr(out), _stream(stream)))


def decode_n_split(g: Geom, n_q_heads: int, n_seq: int, max_len: int, kernel: int = DECODE_AUTO,
                   tiles_per_split: int = 0) -> int:
    r = lib().kvq_decode_n_split(C.byref(g), n_q_heads, n_seq, max_len, kernel, tiles_per_split)
    if r < 0:
        raise KvqError("kvq_decode_n_split", r)
    return r


def decode_partials(g: Geom, q: torch.Tensor, cache: torch.Tensor, seq_byte_off: torch.Tensor, seq_len: torch.Tensor,
                    max_len: int, k_bits: torch.Tensor, k_sigma: torch.Tensor, v_sigma: torch.Tensor,
                    partials: torch.Tensor, softmax_scale: float | None = None, kernel: int = DECODE_AUTO,
                    tiles_per_split: int = 0, stream=None):
    """Split phase only: partials [n_seq, n_q, n_split, 130] fp32 (m in log2 units, l, unnormalised o)."""
    assert q.dtype == torch.float16 and q.is_contiguous() and partials.dtype == torch.float32
    n_seq, n_q = q.shape[0], q.shape[1]
    if softmax_scale is None:
        softmax_scale = g.head_dim ** -0.5
    _check("kvq_decode_partials", lib().kvq_decode_partials(
        C.byref(g), n_q, _ptr(q), _ptr(cache), _ptr(seq_byte_off), _ptr(seq_len), n_seq, max_len, _ptr(k_bits),
        _ptr(k_sigma), _ptr(v_sigma), float(softmax_scale), _ptr(partials), partials.numel() * 4, kernel,
        tiles_per_split, _stream(stream)))


def _step_rows(k_new: torch.Tensor, v_new: torch.Tensor):
    assert k_new.dtype == torch.float16 and v_new.dtype == torch.float16 and k_new.dim() == 3
    assert k_new.stride() == v_new.stride() and k_new.stride(2) == 1
    return k_new.stride(0), k_new.stride(1)


def decode_step_partials(g: Geom, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, cache: torch.Tensor,
                         seq_byte_off: torch.Tensor, seq_len: torch.Tensor, max_len: int, k_bits: torch.Tensor,
                         k_sigma: torch.Tensor, v_sigma: torch.Tensor, partials: torch.Tensor,
                         softmax_scale: float | None = None, kernel: int = DECODE_AUTO, tiles_per_split: int = 0,
                         stream=None):
    """The decode step's split phase: append k_new/v_new [n_seq, n_kv, 128] into slot
    seq_len-1 of each sequence, then partials over all seq_len tokens."""
    assert q.dtype == torch.float16 and q.is_contiguous() and partials.dtype == torch.float32
    ss, sh = _step_rows(k_new, v_new)
    n_seq, n_q = q.shape[0], q.shape[1]
    if softmax_scale is None:
        softmax_scale = g.head_dim ** -0.5
    _check("kvq_decode_step_partials", lib().kvq_decode_step_partials(
        C.byref(g), n_q, _ptr(q), _ptr(k_new), _ptr(v_new), ss, sh, _ptr(cache), _ptr(seq_byte_off), _ptr(seq_len),
        n_seq, max_len, _ptr(k_bits), _ptr(k_sigma), _ptr(v_sigma), float(softmax_scale), _ptr(partials),
        partials.numel() * 4, kernel, tiles_per_split, _stream(stream)))


def decode_step(g: Geom, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, cache: torch.Tensor,
                seq_byte_off: torch.Tensor, seq_len: torch.Tensor, max_len: int, k_bits: torch.Tensor,
                k_sigma: torch.Tensor, v_sigma: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                softmax_scale: float | None = None, kernel: int = DECODE_AUTO, tiles_per_split: int = 0, stream=None):
    """Append the step's token per sequence, then attention (out [n_seq, n_q, 128] fp32)."""
    assert q.dtype == torch.float16 and q.is_contiguous() and out.dtype == torch.float32 and out.is_contiguous()
    ss, sh = _step_rows(k_new, v_new)
    n_seq, n_q = q.shape[0], q.shape[1]
    if softmax_scale is None:
        softmax_scale = g.head_dim ** -0.5
    _check("kvq_decode_step", lib().kvq_decode_step(
        C.byref(g), n_q, _ptr(q), _ptr(k_new), _ptr(v_new), ss, sh, _ptr(cache), _ptr(seq_byte_off), _ptr(seq_len),
        n_seq, max_len, _ptr(k_bits), _ptr(k_sigma), _ptr(v_sigma), float(softmax_scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), kernel, tiles_per_split, _stream(stream)))


def window_workspace_bytes(g: Geom, window: int, n_q_heads: int, n_seq: int, max_len: int,
                           kernel: int = DECODE_AUTO, tiles_per_split: int = 0) -> int:
    r = lib().kvq_window_workspace_bytes(C.byref(g), window, n_q_heads, n_seq, max_len, kernel, tiles_per_split)
    if r < 0:
        raise KvqError("kvq_window_workspace_bytes", r)
    return r


def _window_ring(g: Geom, window: int, win_k: torch.Tensor, win_v: torch.Tensor):
    assert win_k.dtype == torch.float16 and win_v.dtype == torch.float16
    assert win_k.is_contiguous() and win_v.is_contiguous() and win_k.shape == win_v.shape
    assert win_k.shape[1:] == (g.n_kv_heads, window, g.head_dim)


def window_decode_attn(g: Geom, window: int, q: torch.Tensor, win_k: torch.Tensor, win_v: torch.Tensor,
                       cache: torch.Tensor, seq_byte_off: torch.Tensor, seq_len: torch.Tensor, max_len: int,
                       k_bits: torch.Tensor, k_sigma: torch.Tensor, v_sigma: torch.Tensor, out: torch.Tensor,
                       workspace: torch.Tensor, softmax_scale: float | None = None, kernel: int = DECODE_AUTO,
                       tiles_per_split: int = 0, stream=None):
    """Attention over the packed tokens and the fp16 window ring win_k/win_v [n_seq, n_kv, window, 128]."""
    assert q.dtype == torch.float16 and q.is_contiguous() and out.dtype == torch.float32 and out.is_contiguous()
    _window_ring(g, window, win_k, win_v)
    n_seq, n_q = q.shape[0], q.shape[1]
    if softmax_scale is None:
        softmax_scale = g.head_dim ** -0.5
    _check("kvq_window_decode_attn", lib().kvq_window_decode_attn(
        C.byref(g), window, n_q, _ptr(q), _ptr(win_k), _ptr(win_v), _ptr(cache), _ptr(seq_byte_off), _ptr(seq_len),
        n_seq, max_len, _ptr(k_bits), _ptr(k_sigma), _ptr(v_sigma), float(softmax_scale), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), kernel, tiles_per_split, _stream(stream)))


def window_decode_step(g: Geom, window: int, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                       win_k: torch.Tensor, win_v: torch.Tensor, cache: torch.Tensor, seq_byte_off: torch.Tensor,
                       seq_len: torch.Tensor, max_len: int, k_bits: torch.Tensor, k_sigma: torch.Tensor,
                       v_sigma: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                       softmax_scale: float | None = None, kernel: int = DECODE_AUTO, tiles_per_split: int = 0,
                       stream=None):
    """One step with the fp16 window: the token leaving the window is packed, the new one
    enters the ring, attention over all (seq_len counts the new token)."""
    assert q.dtype == torch.float16 and q.is_contiguous() and out.dtype == torch.float32 and out.is_contiguous()
    _window_ring(g, window, win_k, win_v)
    ss, sh = _step_rows(k_new, v_new)
    n_seq, n_q = q.shape[0], q.shape[1]
    if softmax_scale is None:
        softmax_scale = g.head_dim ** -0.5
    _check("kvq_window_decode_step", lib().kvq_window_decode_step(
        C.byref(g), window, n_q, _ptr(q), _ptr(k_new), _ptr(v_new), ss, sh, _ptr(win_k), _ptr(win_v), _ptr(cache),
        _ptr(seq_byte_off), _ptr(seq_len), n_seq, max_len, _ptr(k_bits), _ptr(k_sigma), _ptr(v_sigma),
        float(softmax_scale), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), kernel,
        tiles_per_split, _stream(stream)))


def merge_partials(n_seq: int, n_q: int, n_split: int, partials: torch.Tensor, out: torch.Tensor, stream=None):
    assert partials.dtype == torch.float32 and out.dtype == torch.float32 and out.is_contiguous()
    _check("kvq_merge_partials", lib().kvq_merge_partials(n_seq, n_q, n_split, _ptr(partials), _ptr(out),
                                                          _stream(stream)))


def decode_plan(g: Geom, n_q_heads: int, n_seq: int, max_len: int, kernel: int = DECODE_AUTO,
                tiles_per_split: int = 0) -> dict:
    k, t, n = C.c_int32(), C.c_int32(), C.c_int32()
    w = C.c_int64()
    _check("kvq_decode_plan", lib().kvq_decode_plan(C.byref(g), n_q_heads, n_seq, max_len, kernel, tiles_per_split,
                                                     C.byref(k), C.byref(t), C.byref(n), C.byref(w)))
    return {"kernel": k.value, "tiles_per_split": t.value, "n_split": n.value, "workspace": w.value}


def prefill_plan(g: Geom, n_q_heads: int, n_seq: int, max_q: int, max_len: int, n_split: int = 0) -> dict:
    n, w = C.c_int32(), C.c_int64()
    _check("kvq_prefill_plan", lib().kvq_prefill_plan(C.byref(g), n_q_heads, n_seq, max_q, max_len, n_split,
                                                       C.byref(n), C.byref(w)))
    return {"n_split": n.value, "workspace": w.value}


def prefill_workspace_bytes(g: Geom, n_q_heads: int, n_seq: int, max_q: int, max_len: int, n_split: int = 0) -> int:
    r = lib().kvq_prefill_workspace_bytes(C.byref(g), n_q_heads, n_seq, max_q, max_len, n_split)
    if r < 0:
        raise KvqError("kvq_prefill_workspace_bytes", r)
    return r


def packed_prefill_attn(g: Geom, q: torch.Tensor, cache: torch.Tensor, seq_byte_off: torch.Tensor,
                        q_start: torch.Tensor, n_q: torch.Tensor, max_len: int, k_bits: torch.Tensor,
                        k_sigma: torch.Tensor, v_sigma: torch.Tensor, out: torch.Tensor,
                        workspace: torch.Tensor | None = None, softmax_scale: float | None = None, n_split: int = 0,
                        stream=None):
    """Causal chunk attention: q [n_seq, max_q, n_q_heads, 128] fp16 contiguous -> out (same shape) fp32."""
    assert q.dtype == torch.float16 and q.is_contiguous() and q.dim() == 4
    assert out.dtype == torch.float32 and out.is_contiguous() and out.shape == q.shape
    assert q_start.dtype == torch.int32 and n_q.dtype == torch.int32 and seq_byte_off.dtype == torch.int64
    n_seq, max_q, n_qh = q.shape[0], q.shape[1], q.shape[2]
    if softmax_scale is None:
        softmax_scale = g.head_dim ** -0.5
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("kvq_packed_prefill_attn", lib().kvq_packed_prefill_attn(
        C.byref(g), n_qh, _ptr(q), _ptr(cache), _ptr(seq_byte_off), _ptr(q_start), _ptr(n_q), n_seq, max_q, max_len,
        _ptr(k_bits), _ptr(k_sigma), _ptr(v_sigma), float(softmax_scale), _ptr(out), _ptr(workspace), ws_bytes,
        n_split, _stream(stream)))


ROT_SIGMA_BITS = 0x3DB504F3  # KVQ_ROT_SIGMA_BITS: RN32(1/sqrt(128))


def rot_quantize_pack(g: Geom, k: torch.Tensor, v: torch.Tensor, first_slot: torch.Tensor, n_new: torch.Tensor,
                      src_row0: torch.Tensor, max_new: int, k_signs: torch.Tensor, v_signs: torch.Tensor | None,
                      v_sigma: torch.Tensor | None, cache: torch.Tensor, seq_byte_off: torch.Tensor, stream=None):
    """The rotated variant of quantize_pack (keys, and values when v_signs is given,
    rotated by their KV head's random-sign Walsh-Hadamard transform; uniform widths)."""
    assert k.dtype == torch.float16 and v.dtype == torch.float16 and k.stride() == v.stride() and k.stride(2) == 1
    assert k_signs.dtype == torch.uint8 and (v_signs is None or v_signs.dtype == torch.uint8)
    n_seq = first_slot.shape[0]
    _check("kvq_rot_quantize_pack", lib().kvq_rot_quantize_pack(
        C.byref(g), _ptr(k), _ptr(v), k.stride(0), k.stride(1), n_seq, _ptr(first_slot), _ptr(n_new), _ptr(src_row0),
        max_new, _ptr(k_signs), _ptr(v_signs), _ptr(v_sigma), _ptr(cache), _ptr(seq_byte_off), _stream(stream)))


def rot_queries(g: Geom, q: torch.Tensor, q_rot: torch.Tensor, k_signs: torch.Tensor, stream=None):
    """q [n_seq, n_q, 128] fp16 -> q_rot (same shape), rotated once by the key signs."""
    assert q.dtype == torch.float16 and q.is_contiguous() and q_rot.is_contiguous() and q_rot.dtype == torch.float16
    _check("kvq_rot_queries", lib().kvq_rot_queries(C.byref(g), q.shape[1], q.shape[0], _ptr(q), _ptr(q_rot),
                                                     _ptr(k_signs), _stream(stream)))


def rot_back(g: Geom, out: torch.Tensor, v_signs: torch.Tensor, stream=None):
    """out [n_seq, n_q, 128] fp32, rotated back in place by the value signs."""
    assert out.dtype == torch.float32 and out.is_contiguous()
    _check("kvq_rot_back", lib().kvq_rot_back(C.byref(g), out.shape[1], out.shape[0], _ptr(out), _ptr(v_signs),
                                               _stream(stream)))


def rot_decode_step_partials(g: Geom, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                             cache: torch.Tensor, seq_byte_off: torch.Tensor, seq_len: torch.Tensor, max_len: int,
                             k_bits: torch.Tensor, k_sigma: torch.Tensor, v_sigma: torch.Tensor,
                             k_signs: torch.Tensor, v_signs: torch.Tensor | None, partials: torch.Tensor,
                             softmax_scale: float | None = None, tiles_per_split: int = 0, stream=None):
    """The rotated variant's step split phase in one launch: q [n_seq, n_q, 128] (unrotated)
    rotated inside the attention kernel, the new token [n_seq, n_kv, 128] rotated and packed
    at slot seq_len-1, partials as kvq_decode_partials writes them."""
    assert q.dtype == torch.float16 and q.is_contiguous() and partials.dtype == torch.float32
    ss, sh = _step_rows(k_new, v_new)
    n_seq, n_q = q.shape[0], q.shape[1]
    if softmax_scale is None:
        softmax_scale = g.head_dim ** -0.5
    _check("kvq_rot_decode_step_partials", lib().kvq_rot_decode_step_partials(
        C.byref(g), n_q, _ptr(q), _ptr(k_new), _ptr(v_new), ss, sh, _ptr(cache), _ptr(seq_byte_off), _ptr(seq_len),
        n_seq, max_len, _ptr(k_bits), _ptr(k_sigma), _ptr(v_sigma), _ptr(k_signs), _ptr(v_signs),
        float(softmax_scale), _ptr(partials), partials.numel() * 4, tiles_per_split, _stream(stream)))


def rot_decode_prepare(g: Geom, q: torch.Tensor, q_rot: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                       cache: torch.Tensor, seq_byte_off: torch.Tensor, seq_len: torch.Tensor, k_signs: torch.Tensor,
                       v_signs: torch.Tensor | None, v_sigma: torch.Tensor | None, stream=None):
    """One launch: the new token [n_seq, n_kv, 128] packed (rotated) at slot seq_len - 1, and
    q [n_seq, n_q, 128] rotated into q_rot."""
    assert q.dtype == torch.float16 and q.is_contiguous() and q_rot.is_contiguous() and q_rot.dtype == torch.float16
    ss, sh = _step_rows(k_new, v_new)
    _check("kvq_rot_decode_prepare", lib().kvq_rot_decode_prepare(
        C.byref(g), q.shape[1], q.shape[0], _ptr(q), _ptr(q_rot), _ptr(k_new), _ptr(v_new), ss, sh, _ptr(cache),
        _ptr(seq_byte_off), _ptr(seq_len), _ptr(k_signs), _ptr(v_signs), _ptr(v_sigma), _stream(stream)))


def read_probe(buf: torch.Tensor, sink: torch.Tensor, n_blocks: int, stream=None):
    """Measurement helper: stream-read all of buf (contiguous, 16-byte multiple) once."""
    assert buf.is_contiguous() and sink.dtype == torch.int32 and sink.numel() >= n_blocks
    _check("kvq_read_probe", lib().kvq_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), n_blocks,
                                                   _stream(stream)))
