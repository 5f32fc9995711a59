"""Host checks of the matrix-core Walsh-Hadamard layouts (no GPU).

The quantize kernel for vectors without RoPE and the RoPE-key dequantize
kernel compute H x for 16 vectors as 8 output tiles x 4 K chunks of a
16x16x32 fp16 matrix product, with relabelled coordinates and H's fragments
reduced to two per-lane sign patterns times a tile-uniform sign.  These
tests restate those maps from the kernels' comments and check, lane by lane,
that they multiply by the Sylvester matrix H[i][j] = (-1)^popcount(i & j)
(the Hadamard of the NexusQuant blog, "Handling outliers"), that every
output coordinate lands in exactly one (lane, tile, row) slot, that RoPE
partners share a lane in the dequantize layout, and the exact fp16 encoding
of codeword values the dequantize kernel feeds to the matrix cores.
"""

import numpy as np

N = 128
H = np.array([[(-1) ** bin(i & j).count("1") for j in range(N)] for i in range(N)])


def pc(x):
    return bin(x).count("1")


# quantize (no RoPE): K slot 8p + j of chunk k <- coordinate j + 8k + 32p;
# row m of tile tau -> coordinate (m & 3) + 4 (tau & 1) + 8 (tau >> 1) + 32 (m >> 2)
def q_in(k, p, j):
    return j + 8 * k + 32 * p


def q_out(tau, m):
    return (m & 3) + 4 * (tau & 1) + 8 * (tau >> 1) + 32 * (m >> 2)


def q_frag(tau, k, m, p, j):
    par = pc(m & j & 3) + (tau & 1) * (j >> 2) + pc((m >> 2) & p)
    g = ((tau >> 1) & 1) * (k & 1) + ((tau >> 2) & 1) * (k >> 1)
    return -1 if (par + g) & 1 else 1


# dequantize (RoPE keys): same input map; row m of tile tau -> coordinate
# (m & 7) + 8 (tau & 1) + 16 (tau >> 1 & 1) + 32 (m >> 3) + 64 (tau >> 2)
def d_out(tau, m):
    return (m & 7) + 8 * (tau & 1) + 16 * ((tau >> 1) & 1) + 32 * (m >> 3) + 64 * (tau >> 2)


def d_frag(tau, k, m, p, j):
    par = pc(m & j & 7) + ((m >> 3) & 1) * (p & 1) + (tau >> 2) * (p >> 1)
    g = (tau & 1) * (k & 1) + ((tau >> 1) & 1) * (k >> 1)
    return -1 if (par + g) & 1 else 1


def _product(frag, cout, x):
    """D of every tile from lane-level fragments: lane l = 16p + v supplies A
    row v and B column v at K slots 8p .. 8p+7 (both p = l >> 4)."""
    out = {}
    for tau in range(8):
        D = np.zeros((16, 16))
        for k in range(4):
            A = np.zeros((16, 32))
            B = np.zeros((32, 16))
            for lane in range(64):
                v, p = lane & 15, lane >> 4
                for j in range(8):
                    A[v, 8 * p + j] = frag(tau, k, v, p, j)
                    B[8 * p + j, v] = x[v, q_in(k, p, j)]
            D += A @ B
        out[tau] = D
    return out


def test_fragments_are_hadamard_entries():
    for frag, cout in ((q_frag, q_out), (d_frag, d_out)):
        for tau in range(8):
            for k in range(4):
                for lane in range(64):
                    v, p = lane & 15, lane >> 4
                    for j in range(8):
                        assert frag(tau, k, v, p, j) == H[cout(tau, v), q_in(k, p, j)]


def test_tiles_compute_the_transform_and_cover_every_coordinate():
    x = np.random.default_rng(0).standard_normal((16, N))
    u = x @ H.T
    for frag, cout in ((q_frag, q_out), (d_frag, d_out)):
        D = _product(frag, cout, x)
        seen = np.zeros(N, int)
        for tau in range(8):
            for lane in range(64):
                v, p = lane & 15, lane >> 4
                for r in range(4):
                    c = cout(tau, 4 * p + r)     # lane holds rows 4p .. 4p+3
                    if v == 0:
                        seen[c] += 1
                    assert abs(D[tau][4 * p + r, v] - u[v, c]) < 1e-9
        assert (seen == 1).all()


def test_quantize_lane_holds_four_whole_groups():
    for p in range(4):
        coords = sorted(q_out(tau, 4 * p + r) for tau in range(8) for r in range(4))
        assert coords == list(range(32 * p, 32 * p + 32))
        # element e of group h sits at tile 2h + (e >> 2), row e & 3
        for h in range(4):
            for e in range(8):
                assert q_out(2 * h + (e >> 2), 4 * p + (e & 3)) == 32 * p + 8 * h + e


def test_dequantize_rope_partner_in_same_lane():
    for p in range(4):
        for tau in range(4):
            for r in range(4):
                c = d_out(tau, 4 * p + r)
                assert c < 64 and d_out(tau + 4, 4 * p + r) == c + 64
                # cos / sin index the kernel keeps in registers
                assert c == r + 4 * (p & 1) + 32 * (p >> 1) + 8 * (tau & 1) + 16 * (tau >> 1)


def test_dequantize_codeword_encoding_is_exact():
    """fp16 1024 + 2 idx + c from a group's 16-bit code word, and
    H p = (H (2p + 1028) - 1028 * 128 e_0) / 2 with p = idx - 2 + c/2."""
    rng = np.random.default_rng(1)
    for _ in range(200):
        idx = rng.integers(0, 4, 8)
        c = int(rng.integers(0, 2))
        w = int(sum(int(idx[j]) << (2 * j) for j in range(8)))
        base = 0x64006400 | (0x00010001 if c else 0)
        words = []
        for q in range(4):
            nib = (w >> (4 * q)) & 0xF
            words.append((((nib | (nib << 14)) & 0x00030003) << 1) | base)
        halves = np.array(words, dtype=np.uint32).view(np.uint16).view(np.float16).astype(np.float64)
        np.testing.assert_array_equal(halves, 1024 + 2 * idx + c)
    codes = rng.integers(0, 4, (16, N))
    cos = rng.integers(0, 2, (16, N // 8)).repeat(8, axis=1)
    p = codes - 2 + cos / 2
    enc = (1024 + 2 * codes + cos).astype(np.float64)
    u = enc @ H.T
    assert np.abs(u).max() < 2 ** 24          # every partial sum is an exact fp32 integer
    u[:, 0] -= 1028 * 128
    np.testing.assert_array_equal(u / 2, p @ H.T)
