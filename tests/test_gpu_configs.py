"""GPU parity on the five named workloads at full size.

Caches are compared bit for bit over the whole pool after the step's copies and writes;
decode outputs on a sample of sequences (always including the shortest and the longest),
and prefill-chunk outputs on a sample of rows (always including the first and the last),
are compared with the fp64 oracle within the stated tolerance.
"""

import numpy as np
import pytest

import workloads
from tests.gpu_harness import GpuStep, OracleStep, out_f64, to_raw, tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SAMPLE_SEQS = {1: None, 2: None, 3: 40, 4: 40, 5: 40}


def _sample(lens, k, rng):
    if k is None or k >= len(lens):
        return list(range(len(lens)))
    pick = set(rng.choice(len(lens), size=k, replace=False).tolist())
    pick |= {int(np.argmin(lens)), int(np.argmax(lens))}
    return sorted(pick)


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
    rng = np.random.default_rng(1000 + cfg)
    if c.B:
        seqs = _sample(c.context_lens, SAMPLE_SEQS[cfg], rng)
        got = out_f64(g.out)[seqs]
        want = o.decode(seqs)
        assert np.isfinite(got).all()
        err = np.abs(got - want).max()
        print(f"config {cfg}: decode max abs err {err:.3e} over {len(seqs)} sequences", flush=True)
        assert err <= tol
    if c.chunk is not None:
        total = c.chunk.q.shape[0]
        rows = sorted(set(rng.choice(total, size=min(total, 48), replace=False).tolist()) | {0, total - 1})
        got = out_f64(g.chunk_out)[rows]
        want = o.prefill(rows)[rows]
        assert np.isfinite(got).all()
        err = np.abs(got - want).max()
        print(f"config {cfg}: prefill max abs err {err:.3e} over {len(rows)} rows", flush=True)
        assert err <= tol
