"""Philox counter-based generators, written from their published definition.

Source: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11 (the Philox-N x W-R family).  The pages
name Philox only through the seeded uniforms of the verify step; the key /
counter layout used for the verify step is a reading (see ``verify_uniforms``).

One Philox round on four W-bit words (x0, x1, x2, x3) with key (k0, k1):
    (hi_a, lo_a) = M0 * x0  as a 2W-bit product
    (hi_b, lo_b) = M1 * x2
    new = (hi_b ^ x1 ^ k0, lo_b, hi_a ^ x3 ^ k1, lo_a)
and the key advances by the Weyl increments (W0, W1) between rounds.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
import numpy as np

# Multipliers from the specification; Weyl increments are the fractional parts
# of the golden ratio and of sqrt(3), scaled to W bits (tests re-derive them).
PHILOX4x32 = dict(bits=32, mult=(0xD2511F53, 0xCD9E8D57), weyl=(0x9E3779B9, 0xBB67AE85))
PHILOX4x64 = dict(bits=64, mult=(0xD2E7470EE14C6C93, 0xCA5A826395121157),
                  weyl=(0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B))


def philox_block(counter, key, bits, mult, weyl, rounds=10):
    """One Philox-4xW block on Python integers (any W): returns four W-bit words."""
    mask = (1 << bits) - 1
    x = [int(c) & mask for c in counter]
    k0, k1 = (int(key[0]) & mask, int(key[1]) & mask)
    for r in range(rounds):
        if r:
            k0 = (k0 + weyl[0]) & mask
            k1 = (k1 + weyl[1]) & mask
        pa = mult[0] * x[0]
        pb = mult[1] * x[2]
        x = [(pb >> bits) ^ x[1] ^ k0, pb & mask, (pa >> bits) ^ x[3] ^ k1, pa & mask]
    return tuple(x)


def philox4x32_10(counters, key):
    """Vectorised Philox4x32-10.

    counters: uint32 array [..., 4] (word 0 least significant).
    key:      (k0, k1) 32-bit integers.
    Returns a uint32 array [..., 4].
    """
    c = np.asarray(counters, dtype=np.uint64) & np.uint64(0xFFFFFFFF)
    x0, x1, x2, x3 = (c[..., i].copy() for i in range(4))
    m0, m1 = (np.uint64(v) for v in PHILOX4x32["mult"])
    w0, w1 = PHILOX4x32["weyl"]
    mask = np.uint64(0xFFFFFFFF)
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for r in range(10):
        if r:
            k0 = (k0 + w0) & 0xFFFFFFFF
            k1 = (k1 + w1) & 0xFFFFFFFF
        pa = m0 * x0
        pb = m1 * x2
        x0, x1, x2, x3 = ((pb >> np.uint64(32)) ^ x1 ^ np.uint64(k0), pb & mask,
                          (pa >> np.uint64(32)) ^ x3 ^ np.uint64(k1), pa & mask)
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def verify_uniforms(seed, offset, positions):
    """The two uniforms (u, u') drawn for each verify row.

    READING (the pages give no generator layout): key = (seed low 32 bits,
    seed high 32 bits); counter = (c low 32, c high 32, 0, 0) with
    c = offset + position, where position = b * (gamma + 1) + k is the row's index
    within the call.  u comes from output word 0 and u' from word 1, each as
    (word >> 8) * 2**-24, a value in [0, 1) that float32 holds exactly.
    Returns float64 arrays (u, u_prime) of the positions' shape.
    """
    pos = np.asarray(positions, dtype=np.uint64)
    c = pos + np.uint64(offset)
    ctr = np.stack([c & np.uint64(0xFFFFFFFF), c >> np.uint64(32),
                    np.zeros_like(c), np.zeros_like(c)], axis=-1)
    seed = int(seed) & ((1 << 64) - 1)
    out = philox4x32_10(ctr, (seed & 0xFFFFFFFF, seed >> 32))
    scale = 2.0 ** -24
    u = (out[..., 0] >> np.uint32(8)).astype(np.float64) * scale
    up = (out[..., 1] >> np.uint32(8)).astype(np.float64) * scale
    return u, up


def element_uniforms(seed, offset, position, V):
    """Per-element uniforms U_v, v < V, of one row, for Gumbel-max sampling.

    READING (the pages name the Gumbel-max trick but no generator layout): key as
    in verify_uniforms; counter = (c low 32, c high 32, 1 + v // 4, 0) with
    c = offset + position, output word v % 4; U = ((word >> 8) + 1/2) * 2**-24, in
    (0, 1) strictly, so that -log(-log U) is finite.  Counter word 2 is at least 1,
    so these never coincide with the row's (u, u') (word 2 = 0).
    Returns a float64 array [V].
    """
    c = int(offset) + int(position)
    groups = np.arange((V + 3) // 4, dtype=np.uint64)
    ctr = np.stack([np.full_like(groups, c & 0xFFFFFFFF), np.full_like(groups, (c >> 32) & 0xFFFFFFFF),
                    groups + np.uint64(1), np.zeros_like(groups)], axis=-1)
    seed = int(seed) & ((1 << 64) - 1)
    out = philox4x32_10(ctr, (seed & 0xFFFFFFFF, seed >> 32)).reshape(-1)[:V]
    return ((out >> np.uint32(8)).astype(np.float64) + 0.5) * 2.0 ** -24
