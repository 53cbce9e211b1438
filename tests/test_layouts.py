"""Library layouts of the int4 compressed cache produced by the seeded
generator, checked element by element against the layout the C header
documents (independent of the GPU)."""
import numpy as np

import synthetic as S


def code_at(row, i):
    """Code i of a packed uint8 row: word i // 8, nibble k = (i % 8) // 2 +
    4 ((i % 8) % 2) of that little-endian word (byte k // 2, half k % 2)."""
    j = i % 8
    k = j // 2 + 4 * (j % 2)
    byte = int(row[4 * (i // 8) + k // 2])
    return (byte >> (4 * (k % 2))) & 15


def test_code_word_example():
    # codes 1..8 of one word: bytes c0|c2<<4, c4|c6<<4, c1|c3<<4, c5|c7<<4
    packed = S.pack_codes(np.arange(1, 9))
    assert packed.tolist() == [0x31, 0x75, 0x42, 0x86]


def test_int4_blocked_layouts():
    B, Hkv, cap, D = 2, 2, 96, 64
    g = S.int4_grid(B, Hkv, cap, D, cfg_seed=5)
    kc, vc = g["k_c"], g["v_c"]
    rng = np.random.default_rng(0)
    for _ in range(400):
        b, h = rng.integers(B), rng.integers(Hkv)
        t, d = int(rng.integers(cap)), int(rng.integers(D))
        # k: [cap][D/2], a token's codes in channel order, eight per word
        assert code_at(g["k_codes"][b, h, t], d) == kc[b, h, t, d]
        # v: [cap/32][D][16], per block channel d's 32 codes in token order
        assert code_at(g["v_codes"][b, h, t // 32, d], t % 32) == vc[b, h, t, d]
        # v scale / zero: [cap/32][D/32][32]
        assert g["v_scale"][b, h, t // 32, d // 32, t % 32] == g["v_scale_td"][b, h, t, d // 32]
        assert g["v_zero"][b, h, t // 32, d // 32, t % 32] == g["v_zero_td"][b, h, t, d // 32]
        # k scale / zero: [cap/32][D]
        assert g["k_scale"].shape == (B, Hkv, cap // 32, D)
    assert g["v_codes"].shape == (B, Hkv, cap // 32, D, 16)
    assert g["v_scale"].shape == (B, Hkv, cap // 32, D // 32, 32)


def test_int4_packed_block_layout():
    # one 5120-byte block per 32 tokens: K codes, V codes, K scales, K zeros, V scales, V zeros
    B, Hkv, cap, D = 2, 1, 96, 128
    g = S.int4_grid(B, Hkv, cap, D, cfg_seed=6)
    blk = S.pack_int4_blocks(g["k_codes"], g["v_codes"], g["k_scale"], g["k_zero"], g["v_scale"], g["v_zero"])
    assert blk.shape == (B, Hkv, cap // 32, 5120) and blk.dtype == np.uint8
    u16 = lambda row, off: int(row[off]) | (int(row[off + 1]) << 8)
    rng = np.random.default_rng(1)
    for _ in range(400):
        b, t, d = int(rng.integers(B)), int(rng.integers(cap)), int(rng.integers(D))
        row = blk[b, 0, t // 32]
        j, g32 = t % 32, d // 32
        assert code_at(row[64 * j:64 * j + 64], d) == g["k_c"][b, 0, t, d]
        assert code_at(row[2048 + 16 * d:2048 + 16 * d + 16], j) == g["v_c"][b, 0, t, d]
        assert u16(row, 4096 + 2 * d) == g["k_scale"][b, 0, t // 32, d]
        assert u16(row, 4352 + 2 * d) == g["k_zero"][b, 0, t // 32, d]
        assert u16(row, 4608 + 2 * (32 * g32 + j)) == g["v_scale_td"][b, 0, t, g32]
        assert u16(row, 4864 + 2 * (32 * g32 + j)) == g["v_zero_td"][b, 0, t, g32]
