"""ctypes binding of libpa.so: argument marshalling only.

Every computation runs in the library's HIP kernels.  Tensors are torch tensors on the
current GPU (torch supplies device memory and streams); the binding checks device,
dtype, shape and contiguity, passes raw pointers and the current stream, and raises
PAError for a nonzero status.  If libpa.so has not been built the import of this module
fails: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # loaded first: libpa.so then binds to the HIP runtime torch already loaded

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
PA_DECODE_SHARED_FRAMES = 1
PA_MIXED_SPLIT = 2
PA_MIXED_SEPARATE = 4
DTYPE_CODE = {"f32": PA_F32, "bf16": PA_BF16, "fp8": PA_FP8_E4M3}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
STATUS = {0: "PA_OK", -1: "PA_EINVAL", -2: "PA_ERANGE", -3: "PA_ENOTSUP", -4: "PA_EHIP",
          -5: "PA_ENOSPC"}


class PAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python paged_kv_cache_256_amd/build.py`"
                      " (there is no fallback implementation)")

_lib = ctypes.CDLL(LIB_PATH)

_P, _I, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "pa_last_error": ([], ctypes.c_char_p),
    "pa_build_info": ([], ctypes.c_char_p),
    "pa_reshape_and_cache": ([_P, _P, _P, _P, _P, _I64, _I64, _I, _I, _I, _I, _I, _F, _F, _P], _I),
    "pa_copy_blocks": ([_P, _P, _P, _I64, _I64, _I, _I, _I, _I, _P], _I),
    "pa_decode_workspace_bytes": ([_I, _I, _I, _I, _I, _I], _SZ),
    "pa_decode": ([_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I64, _F, _I, _I, _F, _F, _I,
                   _P, _SZ, _P], _I),
    "pa_decode_ex": ([_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I64, _F, _I, _I, _F, _F, _I,
                      _P, _SZ, ctypes.c_uint, _P], _I),
    "pa_decode_noalloc": ([_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I64, _F, _I, _I, _F,
                           _F, _I, ctypes.c_uint, _P], _I),
    "pa_decode_shared_workspace_bytes": ([_I, _I, _I, _I, _I, _I], _SZ),
    "pa_decode_shared": ([_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I64, _F, _I, _I, _F, _F,
                          _I, _P, _P, _P, _SZ, _P], _I),
    "pa_find_shared_prefixes": ([_P, _I, _P, _I, _I, _I, _P, _P, _P], _I),
    "pa_validate_shared_prefixes": ([_P, _I, _P, _I, _I, _P, _P, _I], _I),
    "pa_prefill_chunk_workspace_bytes": ([_I, _I64, _I, _I, _I, _I, _I, _I, _I], _SZ),
    "pa_prefill_chunk": ([_P, _P, _P, _P, _P, _I, _P, _P, _I, _I64, _I, _I, _I, _I, _I, _I, _I64,
                          _F, _I, _I, _F, _F, _P, _SZ, _P], _I),
    "pa_mixed_workspace_bytes": ([_I, _I, _I64, _I, _I, _I, _I, _I, _I, _I], _SZ),
    "pa_mixed_attention": ([_P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _I64, _I, _I, _I64, _I, _I,
                            _I, _I, _I64, _F, _I, _I, _F, _F, _P, _SZ, ctypes.c_uint, _P], _I),
    "pa_mixed_prefill_units": ([_I, _I, _I64, _I, _I, _I64, _I, _I, _I, _I, _I, ctypes.c_uint], _I),
    "pa_validate_decode_indices": ([_P, _I, _P, _I, _I, _I64, _I], _I),
    "pa_validate_slots": ([_P, _I64, _I64, _I], _I),
    "pa_validate_copy_pairs": ([_P, _I64, _I64], _I),
    "pa_validate_chunk_indices": ([_P, _I, _P, _P, _I, _I, _I64, _I, _I], _I),
    "pa_validate_mixed_indices": ([_P, _I, _P, _P, _I, _I, _I, _I64, _I, _I], _I),
    "pa_bm_create": ([_I64, _I, _P], _I),
    "pa_bm_destroy": ([_P], None),
    "pa_bm_append": ([_P, _P, _I64, _P, _P, _P], _I),
    "pa_bm_append_prompt": ([_P, _I64, _P, _I64, _P, _P], _I),
    "pa_bm_fork": ([_P, _I64, _I64], _I),
    "pa_bm_free": ([_P, _I64], _I),
    "pa_bm_num_free": ([_P, _P], _I),
    "pa_bm_seq_len": ([_P, _I64, _P], _I),
    "pa_bm_ref_count": ([_P, _I64, _P], _I),
    "pa_bm_free_list": ([_P, _P, _I64, _P], _I),
    "pa_bm_block_tables": ([_P, _P, _I64, _P, _I, _P], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)


def lib():
    return _lib


def last_error() -> str:
    return _lib.pa_last_error().decode()


def build_info() -> str:
    return _lib.pa_build_info().decode()


def _check(status: int):
    if status != 0:
        raise PAError(status, last_error())


class PreparedCall:
    """A library call whose arguments were checked and marshalled once (raw device pointers, the
    stream current at preparation).  Calling it issues the same call again; the tensors it was
    prepared from must stay alive and keep their storage."""

    __slots__ = ("_fn", "_args")

    def __init__(self, fn, args):
        self._fn = fn
        self._args = tuple(a if isinstance(a, ctypes._SimpleCData) else t(a)
                           for a, t in zip(args, fn.argtypes))

    def __call__(self):
        status = self._fn(*self._args)
        if status != 0:
            raise PAError(status, last_error())


def _issue(fn, args, prepared: bool):
    if prepared:
        return PreparedCall(fn, args)
    _check(fn(*args))
    return None


def _need_outputs(prepared: bool, **bufs):
    if prepared:
        missing = [k for k, v in bufs.items() if v is None]
        if missing:
            raise ValueError(f"a prepared call needs its {', '.join(missing)} passed in")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _need_rows(t: torch.Tensor, name: str, n: int, exact: bool = True):
    """The index tensor t must have n rows (exact) or at least n rows: the library reads that
    many and trusts the caller for the rest."""
    have = t.shape[0] if t.dim() else 1
    if (have != n) if exact else (have < n):
        raise ValueError(f"{name} has {have} rows, the call needs {'' if exact else 'at least '}{n}")


def _need_out_like(out: torch.Tensor, q: torch.Tensor):
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out must have the shape of q {tuple(q.shape)}, got {tuple(out.shape)}")


def _cache_geometry(k_cache, v_cache, block_size, kv_dtype):
    if k_cache.shape != v_cache.shape or k_cache.dim() != 3:
        raise ValueError("k_cache and v_cache must both be [NB, Hkv, block_size*D]")
    NB, Hkv, tile = k_cache.shape
    if tile % block_size:
        raise ValueError("cache tile size is not a multiple of block_size")
    return NB, Hkv, tile // block_size


def new_kv_cache(NB: int, Hkv: int, block_size: int, D: int, kv_dtype: str, device="cuda"):
    """Empty K and V caches [NB, Hkv, block_size*D] (layout defined in include/pa.h)."""
    shape = (NB, Hkv, block_size * D)
    return (torch.empty(shape, dtype=TORCH_DTYPE[kv_dtype], device=device),
            torch.empty(shape, dtype=TORCH_DTYPE[kv_dtype], device=device))


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, *, block_size: int, kv_dtype: str,
                      k_scale: float = 1.0, v_scale: float = 1.0, prepared: bool = False):
    NB, Hkv, D = _cache_geometry(k_cache, v_cache, block_size, kv_dtype)
    src = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(k.dtype)
    if src is None or v.dtype != k.dtype:
        raise TypeError("k and v must both be float32 or bfloat16")
    T = k.shape[0]
    if tuple(k.shape) != (T, Hkv, D) or tuple(v.shape) != (T, Hkv, D):
        raise ValueError(f"k, v must be [T, {Hkv}, {D}]")
    if slot_mapping.dim() != 1:
        raise ValueError("slot_mapping must be one-dimensional")
    _need_rows(slot_mapping, "slot_mapping", T)
    args = (_dev(k, "k"), _dev(v, "v"), _dev(k_cache, "k_cache", TORCH_DTYPE[kv_dtype]),
            _dev(v_cache, "v_cache", TORCH_DTYPE[kv_dtype]),
            _dev(slot_mapping, "slot_mapping", torch.int64, 1), T, NB, Hkv, D, block_size,
            DTYPE_CODE[src], DTYPE_CODE[kv_dtype], float(k_scale), float(v_scale), _stream(k))
    return _issue(_lib.pa_reshape_and_cache, args, prepared)


def copy_blocks(k_cache, v_cache, pairs, *, block_size: int, kv_dtype: str,
                prepared: bool = False):
    NB, Hkv, D = _cache_geometry(k_cache, v_cache, block_size, kv_dtype)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [N, 2]")
    return _issue(_lib.pa_copy_blocks,
                  (_dev(k_cache, "k_cache", TORCH_DTYPE[kv_dtype]),
                   _dev(v_cache, "v_cache", TORCH_DTYPE[kv_dtype]),
                   _dev(pairs, "pairs", torch.int64), pairs.shape[0], NB, Hkv, D, block_size,
                   DTYPE_CODE[kv_dtype], _stream(k_cache)), prepared)


def decode_workspace_bytes(B, Hq, D, block_size, kv_dtype, max_context_len) -> int:
    return int(_lib.pa_decode_workspace_bytes(B, Hq, D, block_size, DTYPE_CODE[kv_dtype],
                                              max_context_len))


def q_dtype_for(kv_dtype: str) -> str:
    return "f32" if kv_dtype == "f32" else "bf16"


def decode(q, k_cache, v_cache, block_tables, context_lens, *, block_size: int, scale: float,
           kv_dtype: str, max_context_len: int, k_scale: float = 1.0, v_scale: float = 1.0,
           out=None, workspace=None, shared_frames: bool = False, prepared: bool = False):
    """pa_decode_ex; shared_frames=True when frames appear in several sequences' tables (keeps
    them cacheable; the result is bit-identical either way).  prepared=True returns a
    PreparedCall (out and workspace must be given) instead of running the call."""
    _need_outputs(prepared, out=out, workspace=workspace)
    NB, Hkv, D = _cache_geometry(k_cache, v_cache, block_size, kv_dtype)
    qd = q_dtype_for(kv_dtype)
    B, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError(f"q head_dim {Dq} != cache head_dim {D}")
    _need_rows(block_tables, "block_tables", B, exact=False)
    _need_rows(context_lens, "context_lens", B)
    if out is None:
        out = torch.empty_like(q)
    _need_out_like(out, q)
    need = decode_workspace_bytes(B, Hq, D, block_size, kv_dtype, max_context_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if os.environ.get("PA_VALIDATE") == "1":
        validate_decode_indices(block_tables.cpu().numpy(), context_lens.cpu().numpy(),
                                block_size, NB, max_context_len)
    args = (_dev(out, "out", TORCH_DTYPE[qd], 3), _dev(q, "q", TORCH_DTYPE[qd], 3),
            _dev(k_cache, "k_cache", TORCH_DTYPE[kv_dtype]),
            _dev(v_cache, "v_cache", TORCH_DTYPE[kv_dtype]),
            _dev(block_tables, "block_tables", torch.int32, 2), block_tables.shape[1],
            _dev(context_lens, "context_lens", torch.int32, 1), B, Hq, Hkv, D, block_size, NB,
            float(scale), DTYPE_CODE[qd], DTYPE_CODE[kv_dtype], float(k_scale), float(v_scale),
            int(max_context_len), ws, wsb, PA_DECODE_SHARED_FRAMES if shared_frames else 0,
            _stream(q))
    call = _issue(_lib.pa_decode_ex, args, prepared)
    return call if prepared else out


def decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, *, block_size: int,
                   scale: float, kv_dtype: str, max_context_len: int, k_scale: float = 1.0,
                   v_scale: float = 1.0, out=None, shared_frames: bool = False):
    """pa_decode_noalloc: decode with the library's own device scratch instead of a workspace
    (for callers that cannot allocate).  Calls that overlap in time on one GPU must not be
    issued: they share that GPU's scratch."""
    NB, Hkv, D = _cache_geometry(k_cache, v_cache, block_size, kv_dtype)
    qd = q_dtype_for(kv_dtype)
    B, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError(f"q head_dim {Dq} != cache head_dim {D}")
    _need_rows(block_tables, "block_tables", B, exact=False)
    _need_rows(context_lens, "context_lens", B)
    if out is None:
        out = torch.empty_like(q)
    _need_out_like(out, q)
    _check(_lib.pa_decode_noalloc(
        _dev(out, "out", TORCH_DTYPE[qd], 3), _dev(q, "q", TORCH_DTYPE[qd], 3),
        _dev(k_cache, "k_cache", TORCH_DTYPE[kv_dtype]),
        _dev(v_cache, "v_cache", TORCH_DTYPE[kv_dtype]),
        _dev(block_tables, "block_tables", torch.int32, 2), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32, 1), B, Hq, Hkv, D, block_size, NB,
        float(scale), DTYPE_CODE[qd], DTYPE_CODE[kv_dtype], float(k_scale), float(v_scale),
        int(max_context_len), PA_DECODE_SHARED_FRAMES if shared_frames else 0, _stream(q)))
    return out


# Score columns of one run of pa_decode_shared (PA_SHARED_RUN_COLUMNS): a run of s sequences
# needs s * G of them.
SHARED_RUN_COLUMNS = 16


class SharedRuns:
    """Runs of consecutive sequences that share the first frames of their block tables
    (pa_decode_shared): run_size[b] >= 1 starts a run of run_size[b] sequences, 0 marks a
    sequence inside a run; shared_blocks[b] is the table entries b's run shares.  int32 numpy
    arrays (host), or tensors on the decode's device after .to(device)."""

    def __init__(self, shared_blocks, run_size, num_runs: int = 0):
        self.shared_blocks = shared_blocks
        self.run_size = run_size
        self.num_runs = int(num_runs)

    def to(self, device):
        def dv(a):
            return (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(device)
        return SharedRuns(dv(self.shared_blocks), dv(self.run_size), self.num_runs)


def find_shared_prefixes(block_tables, context_lens, block_size: int, max_run: int) -> SharedRuns:
    """pa_find_shared_prefixes on host arrays: the runs of a batch (host numpy arrays)."""
    bt, pbt = _host(block_tables, np.int32)
    cl, pcl = _host(context_lens, np.int32)
    B = cl.shape[0]
    sb = np.zeros(max(B, 1), np.int32)
    rs = np.zeros(max(B, 1), np.int32)
    nr = ctypes.c_int(0)
    _check(_lib.pa_find_shared_prefixes(pbt, bt.shape[1], pcl, B, int(block_size), int(max_run),
                                        ctypes.c_void_p(sb.ctypes.data),
                                        ctypes.c_void_p(rs.ctypes.data), ctypes.byref(nr)))
    return SharedRuns(sb[:B].copy(), rs[:B].copy(), nr.value)


def validate_shared_prefixes(block_tables, context_lens, block_size: int, runs: SharedRuns,
                             G: int):
    bt, pbt = _host(block_tables, np.int32)
    cl, pcl = _host(context_lens, np.int32)
    sb, psb = _host(np.asarray(runs.shared_blocks.cpu() if isinstance(runs.shared_blocks, torch.Tensor)
                               else runs.shared_blocks), np.int32)
    rs, prs = _host(np.asarray(runs.run_size.cpu() if isinstance(runs.run_size, torch.Tensor)
                               else runs.run_size), np.int32)
    if sb.shape[0] != cl.shape[0] or rs.shape[0] != cl.shape[0]:
        raise ValueError("shared_blocks and run_size need one entry per sequence")
    _check(_lib.pa_validate_shared_prefixes(pbt, bt.shape[1], pcl, cl.shape[0], int(block_size),
                                            psb, prs, int(G)))


def decode_shared_workspace_bytes(B, Hq, D, block_size, kv_dtype, max_context_len) -> int:
    return int(_lib.pa_decode_shared_workspace_bytes(B, Hq, D, block_size, DTYPE_CODE[kv_dtype],
                                                     max_context_len))


def decode_shared(q, k_cache, v_cache, block_tables, context_lens, runs: SharedRuns, *,
                  block_size: int, scale: float, kv_dtype: str, max_context_len: int,
                  k_scale: float = 1.0, v_scale: float = 1.0, out=None, workspace=None,
                  prepared: bool = False):
    """pa_decode_shared: decode with each run's shared frames read once for all its members (runs:
    a SharedRuns whose arrays are on q's device)."""
    _need_outputs(prepared, out=out, workspace=workspace)
    NB, Hkv, D = _cache_geometry(k_cache, v_cache, block_size, kv_dtype)
    qd = q_dtype_for(kv_dtype)
    B, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError(f"q head_dim {Dq} != cache head_dim {D}")
    _need_rows(block_tables, "block_tables", B, exact=False)
    _need_rows(context_lens, "context_lens", B)
    _need_rows(runs.shared_blocks, "shared_blocks", B)
    _need_rows(runs.run_size, "run_size", B)
    if out is None:
        out = torch.empty_like(q)
    _need_out_like(out, q)
    need = decode_shared_workspace_bytes(B, Hq, D, block_size, kv_dtype, max_context_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if os.environ.get("PA_VALIDATE") == "1":
        validate_shared_prefixes(block_tables.cpu().numpy(), context_lens.cpu().numpy(),
                                 block_size, runs, Hq // Hkv)
    args = (_dev(out, "out", TORCH_DTYPE[qd], 3), _dev(q, "q", TORCH_DTYPE[qd], 3),
            _dev(k_cache, "k_cache", TORCH_DTYPE[kv_dtype]),
            _dev(v_cache, "v_cache", TORCH_DTYPE[kv_dtype]),
            _dev(block_tables, "block_tables", torch.int32, 2), block_tables.shape[1],
            _dev(context_lens, "context_lens", torch.int32, 1), B, Hq, Hkv, D, block_size, NB,
            float(scale), DTYPE_CODE[qd], DTYPE_CODE[kv_dtype], float(k_scale), float(v_scale),
            int(max_context_len), _dev(runs.shared_blocks, "shared_blocks", torch.int32, 1),
            _dev(runs.run_size, "run_size", torch.int32, 1), ws, wsb, _stream(q))
    call = _issue(_lib.pa_decode_shared, args, prepared)
    return call if prepared else out


def prefill_chunk_workspace_bytes(num_chunks, total_q, max_chunk_len, max_context_len, Hq, Hkv,
                                  D, block_size, kv_dtype) -> int:
    return int(_lib.pa_prefill_chunk_workspace_bytes(num_chunks, total_q, max_chunk_len,
                                                     max_context_len, Hq, Hkv, D, block_size,
                                                     DTYPE_CODE[kv_dtype]))


def prefill_chunk(q, k_cache, v_cache, block_tables, query_start_loc, context_lens, *,
                  block_size: int, scale: float, kv_dtype: str, max_chunk_len: int,
                  max_context_len: int, k_scale: float = 1.0, v_scale: float = 1.0, out=None,
                  workspace=None, prepared: bool = False):
    _need_outputs(prepared, out=out)
    NB, Hkv, D = _cache_geometry(k_cache, v_cache, block_size, kv_dtype)
    qd = q_dtype_for(kv_dtype)
    total_q, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError(f"q head_dim {Dq} != cache head_dim {D}")
    num_chunks = context_lens.shape[0]
    _need_rows(query_start_loc, "query_start_loc", num_chunks + 1)
    _need_rows(block_tables, "block_tables", num_chunks, exact=False)
    if out is None:
        out = torch.empty_like(q)
    _need_out_like(out, q)
    need = prefill_chunk_workspace_bytes(num_chunks, total_q, max_chunk_len, max_context_len, Hq,
                                         Hkv, D, block_size, kv_dtype)
    if need:
        _need_outputs(prepared, workspace=workspace)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if os.environ.get("PA_VALIDATE") == "1":
        validate_chunk_indices(block_tables.cpu().numpy(), query_start_loc.cpu().numpy(),
                               context_lens.cpu().numpy(), block_size, NB, max_chunk_len,
                               max_context_len)
    call = _issue(_lib.pa_prefill_chunk, (
        _dev(out, "out", TORCH_DTYPE[qd], 3), _dev(q, "q", TORCH_DTYPE[qd], 3),
        _dev(k_cache, "k_cache", TORCH_DTYPE[kv_dtype]), _dev(v_cache, "v_cache", TORCH_DTYPE[kv_dtype]),
        _dev(block_tables, "block_tables", torch.int32, 2), block_tables.shape[1],
        _dev(query_start_loc, "query_start_loc", torch.int32, 1),
        _dev(context_lens, "context_lens", torch.int32, 1), num_chunks, total_q, int(max_chunk_len),
        int(max_context_len), Hq, Hkv, D, block_size, NB, float(scale), DTYPE_CODE[qd],
        DTYPE_CODE[kv_dtype], float(k_scale), float(v_scale), ws, wsb, _stream(q)), prepared)
    return call if prepared else out


def mixed_workspace_bytes(num_decodes, num_chunks, total_q, max_chunk_len, max_context_len, Hq,
                          Hkv, D, block_size, kv_dtype) -> int:
    return int(_lib.pa_mixed_workspace_bytes(num_decodes, num_chunks, total_q, max_chunk_len,
                                              max_context_len, Hq, Hkv, D, block_size,
                                              DTYPE_CODE[kv_dtype]))


def _mixed_flags(shared_frames: bool, mode: str) -> int:
    modes = {"auto": 0, "split": PA_MIXED_SPLIT, "separate": PA_MIXED_SEPARATE}
    if mode not in modes:
        raise ValueError(f"mode must be one of {sorted(modes)}")
    return (PA_DECODE_SHARED_FRAMES if shared_frames else 0) | modes[mode]


def mixed_prefill_units(num_decodes, num_chunks, total_q, max_chunk_len, max_context_len,
                        decode_tokens, Hq, Hkv, D, block_size, kv_dtype, mode: str = "auto") -> int:
    """Workgroups a pa_mixed_attention call with these sizes runs prefill tiles on while the
    others stream the decodes (the CU count: separate kernels, or chunks only; 0: decodes only)."""
    return int(_lib.pa_mixed_prefill_units(num_decodes, num_chunks, total_q, max_chunk_len,
                                           max_context_len, int(decode_tokens), Hq, Hkv, D,
                                           block_size, DTYPE_CODE[kv_dtype],
                                           _mixed_flags(False, mode)))


def mixed_attention(q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                    num_decodes: int, *, block_size: int, scale: float, kv_dtype: str,
                    max_chunk_len: int, max_context_len: int, decode_tokens: int = 0,
                    k_scale: float = 1.0, v_scale: float = 1.0, out=None, workspace=None,
                    shared_frames: bool = False, mode: str = "auto", prepared: bool = False):
    """pa_mixed_attention: the first num_decodes sequences are decodes (query row b), the rest
    prefill chunks; one kernel runs both.  decode_tokens (sum of the decodes' context lengths,
    known on the host) and mode ("auto", "split": one kernel runs both halves side by side,
    "separate": the chunk kernels then the decode kernels) only decide how the call uses the
    device."""
    _need_outputs(prepared, out=out)
    NB, Hkv, D = _cache_geometry(k_cache, v_cache, block_size, kv_dtype)
    qd = q_dtype_for(kv_dtype)
    total_q, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError(f"q head_dim {Dq} != cache head_dim {D}")
    num_chunks = context_lens.shape[0] - int(num_decodes)
    if num_chunks < 0 or query_start_loc.shape[0] != context_lens.shape[0] + 1:
        raise ValueError("query_start_loc must have one entry more than context_lens, which "
                         "covers the decodes and the chunks")
    _need_rows(block_tables, "block_tables", context_lens.shape[0], exact=False)
    if out is None:
        out = torch.empty_like(q)
    _need_out_like(out, q)
    need = mixed_workspace_bytes(num_decodes, num_chunks, total_q, max_chunk_len, max_context_len,
                                 Hq, Hkv, D, block_size, kv_dtype)
    if need:
        _need_outputs(prepared, workspace=workspace)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if os.environ.get("PA_VALIDATE") == "1":
        validate_mixed_indices(block_tables.cpu().numpy(), query_start_loc.cpu().numpy(),
                               context_lens.cpu().numpy(), num_decodes, block_size, NB,
                               max_chunk_len, max_context_len)
    call = _issue(_lib.pa_mixed_attention, (
        _dev(out, "out", TORCH_DTYPE[qd], 3), _dev(q, "q", TORCH_DTYPE[qd], 3),
        _dev(k_cache, "k_cache", TORCH_DTYPE[kv_dtype]), _dev(v_cache, "v_cache", TORCH_DTYPE[kv_dtype]),
        _dev(block_tables, "block_tables", torch.int32, 2), block_tables.shape[1],
        _dev(query_start_loc, "query_start_loc", torch.int32, 1),
        _dev(context_lens, "context_lens", torch.int32, 1), int(num_decodes), num_chunks, total_q,
        int(max_chunk_len), int(max_context_len), int(decode_tokens), Hq, Hkv, D, block_size, NB,
        float(scale), DTYPE_CODE[qd], DTYPE_CODE[kv_dtype], float(k_scale), float(v_scale), ws,
        wsb, _mixed_flags(shared_frames, mode), _stream(q)), prepared)
    return call if prepared else out


# ----------------------------------------------------------------------------- host validators


def _host(a, dtype):
    a = np.ascontiguousarray(np.asarray(a, dtype=dtype))
    return a, ctypes.c_void_p(a.ctypes.data)


def validate_decode_indices(block_tables, context_lens, block_size, NB, max_context_len):
    bt, pbt = _host(block_tables, np.int32)
    cl, pcl = _host(context_lens, np.int32)
    _check(_lib.pa_validate_decode_indices(pbt, bt.shape[1], pcl, cl.shape[0], block_size, NB,
                                           int(max_context_len)))


def validate_slots(slot_mapping, NB, block_size):
    s, ps = _host(slot_mapping, np.int64)
    _check(_lib.pa_validate_slots(ps, s.shape[0], NB, block_size))


def validate_copy_pairs(pairs, NB):
    p, pp = _host(np.asarray(pairs).reshape(-1, 2), np.int64)
    _check(_lib.pa_validate_copy_pairs(pp, p.shape[0], NB))


def validate_chunk_indices(block_tables, query_start_loc, context_lens, block_size, NB,
                           max_chunk_len, max_context_len):
    bt, pbt = _host(block_tables, np.int32)
    qs, pqs = _host(query_start_loc, np.int32)
    cl, pcl = _host(context_lens, np.int32)
    _check(_lib.pa_validate_chunk_indices(pbt, bt.shape[1], pqs, pcl, cl.shape[0], block_size, NB,
                                          int(max_chunk_len), int(max_context_len)))


def validate_mixed_indices(block_tables, query_start_loc, context_lens, num_decodes, block_size,
                           NB, max_chunk_len, max_context_len):
    bt, pbt = _host(block_tables, np.int32)
    qs, pqs = _host(query_start_loc, np.int32)
    cl, pcl = _host(context_lens, np.int32)
    nd = int(num_decodes)
    if not 0 <= nd <= cl.shape[0] or qs.shape[0] != cl.shape[0] + 1 or bt.shape[0] != cl.shape[0]:
        raise ValueError("inconsistent mixed-batch index shapes")
    _check(_lib.pa_validate_mixed_indices(pbt, bt.shape[1], pqs, pcl, nd, cl.shape[0] - nd,
                                          block_size, NB, int(max_chunk_len),
                                          int(max_context_len)))


# ----------------------------------------------------------------------------- block manager


class BlockManager:
    """Handle of the library's host-side block manager (pa_bm_* in pa.h): frames, block tables,
    slots and copy-on-write pairs for the GPU calls.  Arguments and results are numpy arrays."""

    def __init__(self, num_frames: int, block_size: int):
        h = ctypes.c_void_p()
        _check(_lib.pa_bm_create(int(num_frames), int(block_size), ctypes.byref(h)))
        self._h = h
        self.num_frames = int(num_frames)
        self.block_size = int(block_size)

    def close(self):
        if self._h:
            _lib.pa_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def append(self, seq_ids):
        """One token per listed id (in order); returns (slots int64 [n], copy_pairs int64 [k, 2])."""
        ids, pids = _host(seq_ids, np.int64)
        ids = ids.reshape(-1)
        n = ids.shape[0]
        slots = np.empty(n, np.int64)
        pairs = np.empty((max(n, 1), 2), np.int64)
        nc = ctypes.c_int64(0)
        _check(_lib.pa_bm_append(self._h, pids, n, ctypes.c_void_p(slots.ctypes.data),
                                 ctypes.c_void_p(pairs.ctypes.data), ctypes.byref(nc)))
        return slots, pairs[:nc.value].copy()

    def append_prompt(self, seq: int, tokens):
        """Start `seq` with prompt token ids; returns (slots int64 [n], cached token count)."""
        t, pt = _host(tokens, np.int32)
        n = t.reshape(-1).shape[0]
        slots = np.empty(n, np.int64)
        cached = ctypes.c_int64(0)
        _check(_lib.pa_bm_append_prompt(self._h, int(seq), pt, n, ctypes.c_void_p(slots.ctypes.data),
                                        ctypes.byref(cached)))
        return slots, cached.value

    def fork(self, parent: int, child: int):
        _check(_lib.pa_bm_fork(self._h, int(parent), int(child)))

    def free(self, seq: int):
        _check(_lib.pa_bm_free(self._h, int(seq)))

    def num_free(self) -> int:
        v = ctypes.c_int64(0)
        _check(_lib.pa_bm_num_free(self._h, ctypes.byref(v)))
        return v.value

    def seq_len(self, seq: int) -> int:
        v = ctypes.c_int64(0)
        _check(_lib.pa_bm_seq_len(self._h, int(seq), ctypes.byref(v)))
        return v.value

    def ref_count(self, frame: int) -> int:
        v = ctypes.c_int32(0)
        _check(_lib.pa_bm_ref_count(self._h, int(frame), ctypes.byref(v)))
        return v.value

    def free_list(self) -> np.ndarray:
        out = np.empty(self.num_frames, np.int32)
        cnt = ctypes.c_int64(0)
        _check(_lib.pa_bm_free_list(self._h, ctypes.c_void_p(out.ctypes.data), self.num_frames,
                                    ctypes.byref(cnt)))
        return out[:cnt.value].copy()

    def block_tables(self, seq_ids, max_blocks_per_seq: int):
        """(tables int32 [n, max_blocks_per_seq] padded with -1, context_lens int32 [n])."""
        ids, pids = _host(seq_ids, np.int64)
        ids = ids.reshape(-1)
        n = ids.shape[0]
        tables = np.empty((n, int(max_blocks_per_seq)), np.int32)
        lens = np.empty(n, np.int32)
        _check(_lib.pa_bm_block_tables(self._h, pids, n, ctypes.c_void_p(tables.ctypes.data),
                                       int(max_blocks_per_seq), ctypes.c_void_p(lens.ctypes.data)))
        return tables, lens
