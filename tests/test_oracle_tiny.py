"""Pins of the tiny decoder and of the loop.

* RoPE against the complex-rotation closed form, RMSNorm against unit RMS.
* One token step against the same architecture composed from torch's own
  float64 primitives (``rms_norm``, ``scaled_dot_product_attention`` with
  ``enable_gqa``, ``silu``).
* The loop: output identical to full-KV greedy decoding ("Riepilogo Tecnico:
  VeriCache", "Risultati Sperimentali"); identity compressor -> every draft
  accepted plus the bonus; k = 0 -> plain greedy steps; the eviction rule keeps
  sinks, the recent window and every 8th older token.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import tiny

RNG = np.random.default_rng(5)


def test_rope_is_complex_rotation():
    D, base = 64, 10000.0
    x = RNG.standard_normal((3, D))
    for pos in (0, 1, 17, 1023, 5000):
        got = tiny.rope(x, pos, base)
        z = x[:, :D // 2] + 1j * x[:, D // 2:]
        theta = base ** (-np.arange(D // 2) * 2.0 / D)
        r = z * np.exp(1j * pos * theta)
        np.testing.assert_allclose(got, np.concatenate([r.real, r.imag], -1), rtol=1e-12, atol=1e-12)


def test_rope_relative_position():
    D = 64
    q = RNG.standard_normal((1, D))
    k = RNG.standard_normal((1, D))
    a = (tiny.rope(q, 100, 1e4) * tiny.rope(k, 90, 1e4)).sum()
    b = (tiny.rope(q, 1010, 1e4) * tiny.rope(k, 1000, 1e4)).sum()
    assert a == pytest.approx(b, rel=1e-9)


def test_rmsnorm_unit_rms():
    x = RNG.standard_normal(256) * 7
    y = tiny.rmsnorm(x, 0.0)
    assert np.sqrt(np.mean(y * y)) == pytest.approx(1.0, rel=1e-14)
    np.testing.assert_allclose(tiny.rmsnorm(x, 1e-5), x / np.sqrt(np.mean(x * x) + 1e-5))


def _torch_step(arrays, spec, token, pos, Kc, Vc):
    """The decoder step composed from torch float64 primitives."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    Hq, Hkv, D = spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    half = D // 2
    theta = spec.rope_base ** (-torch.arange(half, dtype=torch.float64) * 2 / D)
    cos, sin = torch.cos(pos * theta), torch.sin(pos * theta)

    def rot(x):
        return torch.cat([x[..., :half] * cos - x[..., half:] * sin,
                          x[..., half:] * cos + x[..., :half] * sin], -1)

    h = t(arrays["emb"])[token]
    for l in range(spec.n_layers):
        w = {n: t(arrays[f"l{l}.{n}"]) for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")}
        a = F.rms_norm(h, (spec.d_model,), eps=spec.eps)
        q = rot((a @ w["wq"]).view(Hq, 1, D))
        k = rot((a @ w["wk"]).view(Hkv, 1, D))
        v = (a @ w["wv"]).view(Hkv, 1, D)
        K = torch.cat([t(Kc[l]), k], 1)
        V = torch.cat([t(Vc[l]), v], 1)
        o = F.scaled_dot_product_attention(q[None], K[None], V[None], enable_gqa=True)[0]
        h = h + o.reshape(-1) @ w["wo"]
        m = F.rms_norm(h, (spec.d_model,), eps=spec.eps)
        h = h + (F.silu(m @ w["wg"]) * (m @ w["wu"])) @ w["wd"]
    return (F.rms_norm(h, (spec.d_model,), eps=spec.eps) @ t(arrays["w_lm"])).numpy()


def test_token_step_matches_torch_composition(tiny_setup):
    spec, arrays, W, prompt = tiny_setup
    T = 37
    Kc = [RNG.standard_normal((spec.n_kv_heads, T, spec.head_dim)) for _ in range(spec.n_layers)]
    Vc = [RNG.standard_normal((spec.n_kv_heads, T, spec.head_dim)) for _ in range(spec.n_layers)]
    for token, pos in ((3, 37), (511, 900)):
        got, _ = tiny.token_step(W, token, pos, [(Kc[l], Vc[l], None) for l in range(spec.n_layers)])
        ref = _torch_step(arrays, spec, token, pos, Kc, Vc)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_kept_positions_rule():
    kept = tiny.kept_positions(1024)
    assert kept.size == 4 + 111 + 128 == 243
    assert list(kept[:4]) == [0, 1, 2, 3]
    assert list(kept[-128:]) == list(range(896, 1024))
    mid = kept[4:-128]
    assert np.all(mid % 8 == 0) and mid[0] == 8 and mid[-1] == 888
    assert np.all(np.diff(kept) > 0)
    assert tiny.kept_positions(100).tolist() == list(range(100))


def test_loop_equals_greedy_short(tiny_setup):
    spec, arrays, W, prompt = tiny_setup
    ref = tiny.greedy_decode(W, prompt[:160], 24)
    for k in (1, 3, 8):
        toks, rounds = tiny.vericache_decode(
            W, prompt[:160], 24, k, lambda T: tiny.kept_positions(T, 4, 32, 8))
        assert toks == ref
        for r in rounds:
            assert 0 <= r.n <= k and len(r.emitted) == r.n + 1
            assert r.emitted[:r.n] == r.drafts[:r.n]
            if r.n < k:
                assert r.drafts[r.n] != r.predictions[r.n]


def test_identity_compressor_accepts_everything(tiny_setup):
    spec, arrays, W, prompt = tiny_setup
    toks, rounds = tiny.vericache_decode(W, prompt[:96], 20, 4, tiny.all_positions)
    assert toks == tiny.greedy_decode(W, prompt[:96], 20)
    for r in rounds:
        assert r.n == 4 and len(r.emitted) == 5          # all drafts + bonus


def test_k_zero_is_plain_greedy(tiny_setup):
    spec, arrays, W, prompt = tiny_setup
    toks, rounds = tiny.vericache_decode(W, prompt[:64], 6, 0)
    assert toks == tiny.greedy_decode(W, prompt[:64], 6)
    assert all(r.n == 0 and len(r.emitted) == 1 for r in rounds)


@pytest.mark.slow
def test_loop_equals_greedy_full_config(tiny_setup):
    # the measured tiny configuration: prompt 1024, 64 new tokens, k = 8,
    # sinks 4 + last 128 + every 8th older token
    spec, arrays, W, prompt = tiny_setup
    ref = tiny.greedy_decode(W, prompt, 64)
    toks, rounds = tiny.vericache_decode(W, prompt, 64, 8)
    assert toks == ref
    assert sum(len(r.emitted) for r in rounds) >= 63
