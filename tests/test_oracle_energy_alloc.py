"""Pins for the oracle's block energy and greedy allocation.

Page: "RoPE-Aware Bit Allocation for KV-Cache Quantization", abstract -- per layer
and KV head, a label-free energy score per RoPE block; integer widths allocated
greedily by marginal gain under a fixed budget; high-energy blocks get more bits.
Energy is pinned against exact Python integers and invariances of the definition;
the allocation against exhaustive enumeration (the objective sum_i E_i D(b_i) is
separable convex, so greedy marginal allocation is optimal) and its invariants.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle

rng = np.random.default_rng(1234)


def _rand_fp16(shape, scale=1.0, special=True):
    x = (rng.standard_normal(shape) * scale).astype(np.float16)
    if special:
        flat = x.reshape(-1)
        k = min(8, flat.size)
        # subnormals, zeros, signed zeros and the largest finite values
        vals = np.array([6e-8, -6e-8, 0.0, -0.0, 65504.0, -65504.0, 1e-5, -3e-6], np.float16)
        flat[rng.choice(flat.size, k, replace=False)] = vals[:k]
    return x


def _exact_energy(x16, pairing):
    """sum over tokens of k_p^2 + k_q^2, as an exact integer count of 2^-48."""
    n, H, d = x16.shape
    p, q = oracle.coord_map(d, pairing)
    out = np.zeros((H, d // 2), object)
    x = x16.astype(np.float64)  # exact
    for h in range(H):
        for i in range(d // 2):
            s = 0
            for t in range(n):
                for c in (p[i], q[i]):
                    s += int(Fraction(float(x[t, h, c]) ** 2) * (1 << 48))  # x^2 exact in fp64
            out[h, i] = s
    return out


@pytest.mark.parametrize("pairing", [0, 1])
def test_energy_exact_bigint(pairing):
    x = _rand_fp16((37, 3, 16), scale=30.0)
    e = oracle.block_energy(x, pairing)
    ref = _exact_energy(x, pairing)
    assert (oracle.energy_to_int(e) == ref).all()


def test_energy_invariances():
    d = 32
    x = _rand_fp16((50, 2, d), special=False)
    e0 = oracle.energy_to_int(oracle.block_energy(x))
    # token permutation
    e1 = oracle.energy_to_int(oracle.block_energy(x[rng.permutation(50)]))
    assert (e0 == e1).all()
    # rotating each RoPE block by 90 degrees, (a, b) -> (-b, a), is exact in fp16
    y = x.copy()
    y[:, :, : d // 2], y[:, :, d // 2:] = -x[:, :, d // 2:], x[:, :, : d // 2]
    assert (oracle.energy_to_int(oracle.block_energy(y)) == e0).all()
    # scaling by 2^m scales energy by exactly 4^m
    z = (x.astype(np.float32) * 4).astype(np.float16)
    assert (oracle.energy_to_int(oracle.block_energy(z)) == e0 * 16).all()
    # additivity across calls
    acc = oracle.block_energy(x[:20])
    oracle.block_energy(x[20:], energy=acc)
    assert (oracle.energy_to_int(acc) == e0).all()


def test_pairing_is_a_relabelling():
    """Interleaved pairing on permuted coordinates equals half-split on the originals."""
    d = 16
    x = _rand_fp16((20, 1, d), special=False)
    perm = np.empty(d, int)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    eh = oracle.energy_to_int(oracle.block_energy(x, 0))
    ei = oracle.energy_to_int(oracle.block_energy(x[:, :, perm], 1))
    assert (eh == ei).all()


def _energy_from_floats(E):
    """uint64 limb pairs for given non-negative real energies (rounded to 2^-48)."""
    E = np.asarray(E, dtype=object)
    out = np.zeros(E.shape + (2,), np.uint64)
    for idx in np.ndindex(E.shape):
        v = int(Fraction(E[idx]) * (1 << 48))
        out[idx + (0,)] = v & ((1 << 64) - 1)
        out[idx + (1,)] = v >> 64
    return out


def _objective(E_hat, b, Dp):
    return sum(Fraction(e) * Dp[bi] for e, bi in zip(E_hat, b))


def _Dprime():
    """Distortion implied by the binary32 gain table: D'(b) = 1 - sum_{b'<b} dD[b']."""
    dD = [Fraction(float(x)) for x in oracle.tables()["dD"]]
    D = [Fraction(1)]
    for x in dD:
        D.append(D[-1] - x)
    return D


@pytest.mark.parametrize("nb", [1, 2, 3, 4])
def test_greedy_equals_brute_force(nb):
    Dp = _Dprime()
    cases = [rng.exponential(1.0, nb) * 10 ** rng.uniform(-3, 3, nb),
             np.ones(nb), np.zeros(nb), 2.0 ** rng.integers(-8, 8, nb)]
    for E in cases:
        e = _energy_from_floats(E[None, :])
        E_hat = [float(oracle.energy_to_int(e)[0, i]) / 2 ** 48 for i in range(nb)]
        for B in range(0, 8 * nb + 1):
            bits, _ = oracle.allocate(e, B)
            b = [int(v) for v in bits[0]]
            assert sum(b) == B and max(b) <= 8
            best = min(_objective(E_hat, c, Dp)
                       for c in itertools.product(range(9), repeat=nb) if sum(c) == B)
            got = _objective(E_hat, b, Dp)
            assert got == best or abs(float(got - best)) <= 1e-12 * max(float(best), 1e-300)


def test_allocation_invariants():
    nb = 64
    E = rng.exponential(1.0, nb) * np.exp(-np.arange(nb) / 8)
    e = _energy_from_floats(E[None, :])
    for B in (0, 1, 64, 128, 192, 300, 512):
        bits, sig = oracle.allocate(e, B)
        b = bits[0].astype(int)
        assert b.sum() == B and b.max() <= 8
        # more energy never gets fewer bits
        order = np.argsort(-E, kind="stable")
        assert np.all(np.diff(b[order]) <= 0)
        # the per-coordinate scales describe unit-norm keys: 2 * sum sigma^2 = 1
        assert abs(2 * float(np.sum(sig.astype(np.float64) ** 2)) - 1) < 1e-6
    # scaling every energy by 4^m leaves widths and scales unchanged
    b1, s1 = oracle.allocate(e, 192)
    b2, s2 = oracle.allocate(_energy_from_floats((E * 16)[None, :]), 192)
    assert (b1 == b2).all() and (s1 == s2).all()


def test_equal_energies_give_uniform_and_modes():
    e = _energy_from_floats(np.full((2, 64), 3.0))
    for B in (64, 128, 192):
        g, sg = oracle.allocate(e, B, oracle.GREEDY)
        u, su = oracle.allocate(e, B, oracle.UNIFORM)
        assert (g == B // 64).all() and (u == B // 64).all()
        assert np.allclose(sg, 1 / np.sqrt(128)) and (sg == su).all()
    # fp16 passthrough: every block 16
    p, _ = oracle.allocate(e, 16 * 64)
    assert (p == 16).all()
    # zero energy: scales are 0
    b, s = oracle.allocate(_energy_from_floats(np.zeros((1, 64))), 128)
    assert (s == 0).all() and b.sum() == 128


def test_invalid_budgets():
    e = _energy_from_floats(np.ones((1, 64)))
    for B in (-1, 513, 1000):
        with pytest.raises(ValueError):
            oracle.allocate(e, B)
    with pytest.raises(ValueError):
        oracle.allocate(e, 100, oracle.UNIFORM)


def test_cap_binds_on_steep_spectrum():
    """Energies spanning 1e10 force the 8-bit cap on the top blocks."""
    E = 10.0 ** (-np.arange(64) / 6.4)
    bits, _ = oracle.allocate(_energy_from_floats(E[None, :]), 192)
    assert bits[0, 0] == 8 and (bits[0] == 0).sum() > 10
