"""GPU parity on the five named workloads at full size, every output compared.

Caches are compared bit for bit over the whole pool after the step's copies and writes.  Every
decode output (all B sequences, all query heads) and every prefill-chunk row is compared with the
fp64 oracle within the stated tolerance; the per-config maximum absolute error is printed.
"""

import time

import numpy as np
import pytest

import workloads
from tests.gpu_harness import GpuStep, OracleStep, out_f64, to_raw, tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_named_config(cfg):
    print(f"config {cfg}: generating", flush=True)
    c = workloads.make(cfg)
    g = GpuStep(c)
    g.step()
    print(f"config {cfg}: gpu step done, building oracle caches", flush=True)
    o = OracleStep(c)
    np.testing.assert_array_equal(to_raw(g.kc), o.kc)
    np.testing.assert_array_equal(to_raw(g.vc), o.vc)
    print(f"config {cfg}: caches bit-exact ({c.NB} frames)", flush=True)
    tol = tolerance(c)
    if c.B:
        t0 = time.time()
        got = out_f64(g.out)
        want = o.decode()
        assert got.shape == want.shape == (c.B, c.q.shape[1], c.D)
        assert np.isfinite(got).all()
        err = np.abs(got - want).max()
        print(f"config {cfg}: decode max abs err {err:.3e} over all {c.B} sequences "
              f"(oracle {time.time() - t0:.1f}s)", flush=True)
        assert err <= tol
    if c.chunk is not None:
        t0 = time.time()
        got = out_f64(g.chunk_out)
        want = o.prefill()
        assert np.isfinite(got).all()
        err = np.abs(got - want).max()
        print(f"config {cfg}: prefill max abs err {err:.3e} over all {got.shape[0]} rows "
              f"(oracle {time.time() - t0:.1f}s)", flush=True)
        assert err <= tol


@pytest.mark.parametrize("n", [1, 4, 16])
def test_long_context_decode(n):
    """n sequences of 32,768 tokens at the 70B layer shape: each (sequence, kv head) run is cut
    into many wavefront ranges and merged from partials; every output against the oracle."""
    print(f"long context: {n} x 32768 tokens, generating", flush=True)
    c = workloads.long_context(n)
    g = GpuStep(c)
    g.step()
    o = OracleStep(c)
    np.testing.assert_array_equal(to_raw(g.kc), o.kc)
    np.testing.assert_array_equal(to_raw(g.vc), o.vc)
    got = out_f64(g.out)
    assert np.isfinite(got).all()
    err = np.abs(got - o.decode()).max()
    print(f"long context {n}: decode max abs err {err:.3e} over all outputs", flush=True)
    assert err <= tolerance(c)
