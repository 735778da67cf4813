"""pa_decode_noalloc, the decode entry point that allocates nothing (its plan and partials live in
the library's per-GPU scratch array), called through the C ABI and compared with pa_decode_ex on
a workspace: bit-identical outputs, and within the oracle's tolerance, on two calls in a row with
the second batch smaller than the first (the scratch keeps the first call's contents)."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_256_amd as pa
import workloads
from paged_kv_cache_256_amd._binding import DTYPE_CODE
from tests.gpu_harness import GpuStep, OracleStep, out_f64, tolerance

pytestmark = pytest.mark.gpu


def _noalloc(g: GpuStep, out: torch.Tensor) -> int:
    c = g.c
    f = pa.lib().pa_decode_noalloc
    qd = DTYPE_CODE[pa.q_dtype_for(c.kv_dtype)]
    P = ctypes.c_void_p
    return f(P(out.data_ptr()), P(g.q.data_ptr()), P(g.kc.data_ptr()), P(g.vc.data_ptr()),
             P(g.tables.data_ptr()), g.tables.shape[1], P(g.lens.data_ptr()), c.B, c.q.shape[1],
             c.Hkv, c.D, c.bs, c.NB, ctypes.c_float(c.scale), qd, DTYPE_CODE[c.kv_dtype],
             ctypes.c_float(c.k_scale), ctypes.c_float(c.v_scale), c.max_context_len,
             ctypes.c_uint(1 if c.shares_frames else 0),
             P(torch.cuda.current_stream().cuda_stream))


CALLS = [
    # the second call is smaller: fewer sequences, shorter contexts, fewer heads
    ("first", 301, dict(Hq=64, Hkv=8, D=128, bs=16, kv_dtype="bf16",
                        lens=[1, 16, 17, 300, 2048, 4100, 9000, 800] * 6)),
    ("second, smaller", 302, dict(Hq=8, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                                  lens=[5, 33, 700])),
]


def test_noalloc_decode_matches_the_workspace_call_twice_in_a_row():
    results = []
    for name, seed, kw in CALLS:
        print(f"pa_decode_noalloc: {name} call, {len(kw['lens'])} sequences", flush=True)
        lens = kw.pop("lens")
        c = workloads.decode_case("noalloc", seed, lens=lens, std=0.7071, pool="scattered", **kw)
        kw["lens"] = lens
        g = GpuStep(c)
        g.write()
        ref = g.decode().clone()  # pa_decode_ex with its own workspace
        out = torch.full_like(ref, float("nan"))
        status = _noalloc(g, out)
        assert status == 0, pa.last_error()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), \
            f"{name}: pa_decode_noalloc differs from pa_decode_ex"
        err = np.abs(out_f64(out) - OracleStep(c).decode()).max()
        print(f"  bit-identical to pa_decode_ex; max abs err against the oracle {err:.2e}",
              flush=True)
        assert err <= tolerance(c)
        results.append(err)
    assert len(results) == 2
