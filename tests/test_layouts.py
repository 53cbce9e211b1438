"""Library layouts of the int4 compressed cache produced by the seeded
generator, checked element by element against the layout the C header
documents (independent of the GPU)."""
import numpy as np

import synthetic as S


def test_int4_blocked_layouts():
    B, Hkv, cap, D = 2, 2, 96, 64
    g = S.int4_grid(B, Hkv, cap, D, cfg_seed=5)
    kc, vc = g["k_c"], g["v_c"]
    rng = np.random.default_rng(0)
    for _ in range(400):
        b, h = rng.integers(B), rng.integers(Hkv)
        t, d = int(rng.integers(cap)), int(rng.integers(D))
        # k: [cap][D/2], two channels per byte, even channel in the low nibble
        byte = int(g["k_codes"][b, h, t, d // 2])
        assert (byte >> (4 * (d & 1))) & 15 == kc[b, h, t, d]
        # v: [cap/32][D][16], per block channel d's 32 tokens, even token low
        byte = int(g["v_codes"][b, h, t // 32, d, (t % 32) // 2])
        assert (byte >> (4 * (t & 1))) & 15 == vc[b, h, t, d]
        # v scale / zero: [cap/32][D/32][32]
        assert g["v_scale"][b, h, t // 32, d // 32, t % 32] == g["v_scale_td"][b, h, t, d // 32]
        assert g["v_zero"][b, h, t // 32, d // 32, t % 32] == g["v_zero_td"][b, h, t, d // 32]
        # k scale / zero: [cap/32][D]
        assert g["k_scale"].shape == (B, Hkv, cap // 32, D)
    assert g["v_codes"].shape == (B, Hkv, cap // 32, D, 16)
    assert g["v_scale"].shape == (B, Hkv, cap // 32, D // 32, 32)
