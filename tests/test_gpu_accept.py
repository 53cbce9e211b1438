"""GPU parity of vc_accept (argmax + accept-until-first-mismatch) against the
oracle, bit-exact, on planted acceptance patterns, forced ties and edge cases."""
import numpy as np
import pytest

import synthetic as S
from oracle.accept import accept_batch
from oracle.formats import bf16_to_f64

from .helpers import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _run(logits_np, drafts, dtype):
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    if dtype == "bf16":
        bits = S.f32_to_bf16_bits(logits_np)
        lg = to_dev_bf16(bits)
        ref_logits = bf16_to_f64(bits)
    else:
        lg = to_dev(logits_np.astype(np.float32))
        ref_logits = logits_np.astype(np.float64)
    d = to_dev(drafts.astype(np.int32).reshape(drafts.shape[0], -1))
    am, n, toks, n_out = vc.accept(lg, d)
    torch.cuda.synchronize()
    ref = accept_batch(ref_logits, drafts)
    got = [t.cpu().numpy() for t in (am, n, toks, n_out)]
    for g, r, name in zip(got, ref, ("argmax", "accept_len", "out_tokens", "n_out")):
        np.testing.assert_array_equal(g, r, err_msg=name)
    return got


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("V", [32768, 1000, 513])
def test_planted_patterns(dtype, V):
    B, k = 16, 32
    y, d, n = S.planted_accept(B, k, V, cfg_seed=4, n_lo=24, n_hi=32, force={0: 0, 1: k, 2: 1})
    logits = S.planted_logits(y, V, cfg_seed=4)
    got = _run(logits, d, dtype)
    np.testing.assert_array_equal(got[1], n)           # planted accept lengths recovered
    assert got[1][1] == k and got[3][1] == k + 1       # full match -> bonus
    assert got[1][0] == 0 and got[3][0] == 1           # first-position mismatch


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_forced_ties_lowest_index(dtype):
    B, k, V = 8, 8, 4096
    y, d, n = S.planted_accept(B, k, V, cfg_seed=11, n_lo=0, n_hi=k)
    logits = S.planted_logits(y, V, cfg_seed=11, ties=5)
    _run(logits, d, dtype)


def test_small_integer_logits_many_ties():
    rng = np.random.default_rng(3)
    logits = rng.integers(-2, 3, (5, 9, 77)).astype(np.float32)
    drafts = rng.integers(0, 3, (5, 8)).astype(np.int32)
    _run(logits, drafts, "fp32")
    _run(logits, drafts, "bf16")


def test_k0_and_long_block():
    rng = np.random.default_rng(4)
    # M = 1: one greedy step, no drafts
    logits = rng.standard_normal((3, 1, 300)).astype(np.float32)
    _run(logits, np.zeros((3, 0), np.int32), "fp32")
    # M = 100 > 64: the first mismatch may lie beyond one wave's ballot
    y, d, n = S.planted_accept(4, 99, 512, cfg_seed=5, n_lo=70, n_hi=99, force={3: 99})
    got = _run(S.planted_logits(y, 512, cfg_seed=5), d, "fp32")
    np.testing.assert_array_equal(got[1], n)


def test_negative_zero_equals_positive_zero():
    logits = np.zeros((1, 2, 16), np.float32)
    logits[0, 0, :] = -1
    logits[0, 0, 3] = -0.0
    logits[0, 0, 5] = 0.0
    _run(logits, np.array([[3]], np.int32), "fp32")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_planted_patterns_1m_config(dtype):
    # the 1M-token configuration's block: k = 40 drafts (M = 41) over a 131072-token vocabulary;
    # the full-accept + bonus and the first-position-mismatch patterns and one n ~ U{24..40}
    B, k, V = 3, 40, 131072
    y, d, n = S.planted_accept(B, k, V, cfg_seed=5, n_lo=24, n_hi=40, force={0: k, 1: 0})
    got = _run(S.planted_logits(y, V, cfg_seed=5), d, dtype)
    np.testing.assert_array_equal(got[1], n)
    assert got[1][0] == k and got[3][0] == k + 1
    assert got[1][1] == 0 and got[3][1] == 1
