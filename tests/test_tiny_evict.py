"""CPU checks of the tiny loop's eviction compressor in libvc: the kept
count that vc_evict_kept_count computes in closed form equals the size of
the oracle's kept set for every committed length and several rules (sinks,
recent window, stride; the identity rule is sinks 0, recent 0, stride 1), and
vc_gather_evict rejects a compacted cache too small for a full source cache
before any GPU work."""
import ctypes

import pytest

from oracle import tiny


@pytest.fixture(scope="module")
def L():
    from lossless_speculative_decoding_vc_amd import build as vbuild
    import os
    if not os.path.exists(vbuild.LIB):
        vbuild.build()
    from lossless_speculative_decoding_vc_amd.tiny_loop import _setup_lib
    return _setup_lib()


@pytest.mark.parametrize("rule", [(4, 128, 8), (4, 32, 8), (0, 16, 5), (7, 0, 3), (0, 0, 1), (3, 5, 1), (2, 9, 64)])
def test_kept_count_equals_the_oracle_rule(L, rule):
    for T in list(range(0, 300)) + [511, 512, 1023, 1024, 1025, 4096, 65537]:
        assert L.vc_evict_kept_count(T, *rule) == len(tiny.kept_positions(T, *rule)), (T, rule)


def test_kept_count_rejects_bad_rules(L):
    assert L.vc_evict_kept_count(10, 4, 4, 0) == -1
    assert L.vc_evict_kept_count(-1, 4, 4, 8) == -1
    assert L.vc_evict_kept_count(10, -1, 4, 8) == -1


def test_gather_evict_checks_capacity_on_the_host(L):
    import lossless_speculative_decoding_vc_amd as vc
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: every case fails validation
    need = L.vc_evict_kept_count(1088, 4, 128, 8)
    small = (need // 32) * 32 if need % 32 else need - 32
    args = lambda dcap, stride=8: (2, 64, fake, 4, 128, stride, fake, fake, 1088, fake, fake, dcap, fake, None)
    assert L.vc_gather_evict(*args(small)) == vc.VC_EINVAL
    assert b"cannot hold" in L.vc_last_error()
    assert L.vc_gather_evict(*args(need + 1)) == vc.VC_EINVAL          # not a multiple of 32
    assert L.vc_gather_evict(*args((need + 31) // 32 * 32, stride=0)) == vc.VC_EINVAL
