"""The C ABI called from several host threads at once (CPU; validation paths and the host-side
offline split only, no GPU): every thread gets the result a single-threaded call gives.  The
library keeps no state between calls, so concurrent calls must not interfere."""

import threading

import numpy as np
import pytest

import w4a4_bit_quantized_amd as w4
from w4a4_bit_quantized_amd import binding

P = 0x10000  # a fake, well-aligned device address; the validation paths never dereference it


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(binding.library_path()):
        from w4a4_bit_quantized_amd import build
        build.build()
    return w4.load_library()


def _calls(lib):
    """(call, expected status) pairs covering every entry point's validation."""
    return [
        (lambda: lib.svdq_quantize_act(P, P, P, 16, 40, 8, 0, P, P, P, None), 2),
        (lambda: lib.svdq_quantize_act(P, P, None, 16, 64, 8, 0, P, P, P, None), 1),
        (lambda: lib.svdq_quantize_act(P, P, P, 0, 64, 8, 0, P, P, P, None), 0),
        (lambda: lib.svdq_quantize_weight(P, P, 8, 64, 12, P, P, None), 4),
        (lambda: lib.svdq_gemm_lowrank(P + 8, P, P, P, P, P, P, P, 16, 16, 64, 8, P, None), 3),
        (lambda: lib.svdq_gemm_lowrank_mx(P, P, P, P, P, P, P, P, 16, 18, 128, 8, P, None), 2),
        (lambda: lib.svdq_linear(P, P, P, P, P, P, P, P, 16, 16, 64, 8, 0, P, P, 1, None), 2),
        (lambda: lib.svdq_linear_mx(P, P, P, P, P, P, P, P, 16, 16, 64, 8, 64, P, P, 1 << 20, None), 4),
        (lambda: lib.w4a4_hadamard_transform(P, 64, P, 64, 4, 64, 3, 0, None), 4),
        (lambda: int(lib.svdq_linear_workspace_bytes(4096, 3072, 32) > 0), 1),
    ]


def test_validation_from_many_threads(lib):
    calls = _calls(lib)
    for f, want in calls:
        assert f() == want
    errors = []

    def worker(seed):
        rng = np.random.default_rng(seed)
        for i in rng.integers(0, len(calls), 2000):
            f, want = calls[i]
            got = f()
            if got != want:
                errors.append((i, got, want))

    threads = [threading.Thread(target=worker, args=(s,)) for s in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:5]


def test_lowrank_split_from_many_threads(lib):
    """Four concurrent offline splits (each itself multi-threaded) equal the sequential ones."""
    rng = np.random.default_rng(3)
    from oracle import formats
    jobs = []
    for s in range(4):
        w = formats.bf16_from_f64(rng.standard_normal((48, 40)) / 8)
        lam = formats.bf16_from_f64(rng.uniform(0.5, 2.0, 40))
        jobs.append((w, lam, s))
    ref = [w4.svdq_lowrank_split(w, lam, 6, seed=s, threads=2) for w, lam, s in jobs]
    out = [None] * len(jobs)

    def worker(j):
        w, lam, s = jobs[j]
        out[j] = w4.svdq_lowrank_split(w, lam, 6, seed=s, threads=2)

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for a, b in zip(ref, out):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
