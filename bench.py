"""Benchmark of the paged-attention hot path on one MI355X.

Default workload: the Llama-3-70B-shaped decode layer (256 sequences, 64 query heads, 8 KV
heads, head_dim 128, bf16, 16-token blocks, context lengths log-uniform in [128, 8192] over a
scattered pool).  One step = pa_reshape_and_cache of the step's 256 new tokens + pa_decode
(plan, stream and reduce kernels), on inputs resident in HBM.  Before every timed step a 512 MiB
buffer is read so the KV cache does not sit in L2 / the MALL from the previous step (a decode
layer's KV is evicted by the other layers of a model in practice); the eviction is a read so that
no dirty lines are written back inside the timed region.

Prints ONE JSON line.  `value` is the KV GB/s of the whole step (algorithmic KV bytes / step
time); seqs/s per layer, the roofline of the decode kernels and the CPU oracle's rate on a
bounded sample are reported beside it.  --config N benches another of the five workloads
(same fields); --gpus N>1 is refused (single-GPU build).
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
METRIC = "paged-attn decode KV GB/s (% of HBM peak) + seqs/s, 70B-shape layer, 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def measured_traffic(workload: str):
    """HBM bytes per pa_decode call from the committed counter summary of this workload, if the
    decode kernel sources are unchanged since the counters were taken (else None)."""
    import glob
    import hashlib

    for path in glob.glob(os.path.join(ROOT, "profiles", "*_traffic.txt")):
        try:
            doc = json.load(open(path))
        except (OSError, ValueError):
            continue
        if doc.get("workload") != workload:
            continue
        h = hashlib.sha256()
        for src in doc["kernel_sources"]:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() == doc["kernel_sources_sha256"]:
            return int(doc["traffic_bytes_per_call"]), os.path.relpath(path, ROOT)
    return None


def chunk_flops(case) -> int:
    """4 * D * Hq * sum_i (pos_i + 1): QK^T and P.V over the causal key ranges, 2 FLOP per MAC."""
    ch = case.chunk
    total = 0
    for c in range(ch.num_chunks):
        C = int(ch.query_start_loc[c + 1] - ch.query_start_loc[c])
        L = int(ch.context_lens[c])
        pos = np.arange(L - C, L, dtype=np.int64)
        total += int((pos + 1).sum())
    return 4 * case.D * case.Hq * total


class DeviceState:
    """A workload's device buffers: the KV caches (filled once over every pool slot), the
    step's inputs, and preallocated outputs and workspaces, so a step allocates nothing."""

    def __init__(self, case, dev):
        import torch

        import paged_kv_cache_256_amd as pa

        self.c = c = case
        self.pa = pa

        def dv(a, kind):
            a = np.ascontiguousarray(a)
            if kind == "bf16":
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        s = c.src_dtype
        self.kc, self.vc = pa.new_kv_cache(c.NB, c.Hkv, c.bs, c.D, c.kv_dtype, device=dev)
        pk, pv = dv(c.pool_k, s), dv(c.pool_v, s)
        slots = torch.arange(c.NB * c.bs, dtype=torch.int64, device=dev)
        pa.reshape_and_cache(pk, pv, self.kc, self.vc, slots, block_size=c.bs,
                             kv_dtype=c.kv_dtype, k_scale=c.k_scale, v_scale=c.v_scale)
        del pk, pv, slots
        self.new_k, self.new_v = dv(c.new_k, s), dv(c.new_v, s)
        self.new_slots = dv(c.new_slots, "i64")
        self.pairs = dv(c.copy_pairs, "i64") if len(c.copy_pairs) else None
        if c.B:
            self.q = dv(c.q, c.q_dtype)
            self.tables = dv(c.block_tables, "i32")
            self.lens = dv(c.context_lens, "i32")
            self.out = torch.empty_like(self.q)
            need = pa.decode_workspace_bytes(c.B, c.Hq, c.D, c.bs, c.kv_dtype, c.max_context_len)
            self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            self.groups = None
            # the caller's cache-policy hint: do several sequences' tables name the same frame?
            self.shared = c.shares_frames
        if c.chunk is not None:
            ch = c.chunk
            self.cq = dv(ch.q, c.q_dtype)
            self.ctables = dv(ch.block_tables, "i32")
            self.cqsl = dv(ch.query_start_loc, "i32")
            self.clens = dv(ch.context_lens, "i32")
            self.cout = torch.empty_like(self.cq)
            need = pa.prefill_chunk_workspace_bytes(
                ch.num_chunks, self.cq.shape[0], ch.max_chunk_len, ch.max_context_len, c.Hq,
                c.Hkv, c.D, c.bs, c.kv_dtype)
            self.cws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def init_mixed(self, dev, mode="auto"):
        """Inputs of pa_mixed_attention: the decodes and the chunks as one batch (decodes first)."""
        import torch

        import workloads

        c, pa = self.c, self.pa
        m = self.m = workloads.mixed_batch(c)
        self.mq = (torch.from_numpy(np.ascontiguousarray(m.q).view(np.int16)).to(dev).view(torch.bfloat16)
                   if c.q_dtype == "bf16" else torch.from_numpy(np.ascontiguousarray(m.q)).to(dev))
        self.mtables = torch.from_numpy(m.block_tables).to(dev)
        self.mqsl = torch.from_numpy(m.query_start_loc).to(dev)
        self.mlens = torch.from_numpy(m.context_lens).to(dev)
        self.mout = torch.empty_like(self.mq)
        need = pa.mixed_workspace_bytes(m.num_decodes, c.chunk.num_chunks, self.mq.shape[0],
                                        m.max_chunk_len, m.max_context_len, c.Hq, c.Hkv, c.D,
                                        c.bs, c.kv_dtype)
        self.mws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        self.mixed_units = pa.mixed_prefill_units(m.num_decodes, c.chunk.num_chunks,
                                                  self.mq.shape[0], m.max_chunk_len,
                                                  m.max_context_len, m.decode_tokens, c.Hq, c.Hkv,
                                                  c.D, c.bs, c.kv_dtype, mode)
        self.mixed_mode = mode

    def mixed(self, prepared=False):
        c, m = self.c, self.m
        return self.pa.mixed_attention(self.mq, self.kc, self.vc, self.mtables, self.mqsl, self.mlens,
                                m.num_decodes, block_size=c.bs, scale=c.scale,
                                kv_dtype=c.kv_dtype, max_chunk_len=m.max_chunk_len,
                                max_context_len=m.max_context_len, decode_tokens=m.decode_tokens,
                                k_scale=c.k_scale, v_scale=c.v_scale, out=self.mout,
                                workspace=self.mws, shared_frames=self.shared,
                                mode=self.mixed_mode, prepared=prepared)

    def write(self, prepared=False):
        c, pa = self.c, self.pa
        calls = []
        if self.pairs is not None:
            calls.append(pa.copy_blocks(self.kc, self.vc, self.pairs, block_size=c.bs,
                                        kv_dtype=c.kv_dtype, prepared=prepared))
        calls.append(pa.reshape_and_cache(self.new_k, self.new_v, self.kc, self.vc,
                                          self.new_slots, block_size=c.bs, kv_dtype=c.kv_dtype,
                                          k_scale=c.k_scale, v_scale=c.v_scale,
                                          prepared=prepared))
        if prepared:
            def both():
                for f in calls:
                    f()
            return both

    def prefill(self, prepared=False):
        c, ch = self.c, self.c.chunk
        return self.pa.prefill_chunk(self.cq, self.kc, self.vc, self.ctables, self.cqsl, self.clens,
                              block_size=c.bs, scale=c.scale, kv_dtype=c.kv_dtype,
                              max_chunk_len=ch.max_chunk_len, max_context_len=ch.max_context_len,
                              k_scale=c.k_scale, v_scale=c.v_scale, out=self.cout,
                              workspace=self.cws, prepared=prepared)

    def init_shared(self, dev, max_run=None):
        """Runs of consecutive sequences that share their tables' first frames (found on the host,
        like the block tables a scheduler hands over) for pa_decode_shared: at most max_run
        sequences a run (default: as many as the run's score columns hold)."""
        c, pa = self.c, self.pa
        import torch

        most = max(1, pa.SHARED_RUN_COLUMNS // (c.Hq // c.Hkv))
        r = pa.find_shared_prefixes(c.block_tables, c.context_lens, c.bs,
                                    min(most, max_run) if max_run else most)
        self.groups = r.to(dev)
        need = pa.decode_shared_workspace_bytes(c.B, c.Hq, c.D, c.bs, c.kv_dtype, c.max_context_len)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        return r

    def decode(self, prepared=False):
        c = self.c
        if self.groups is not None:
            return self.pa.decode_shared(self.q, self.kc, self.vc, self.tables, self.lens,
                                         self.groups, block_size=c.bs, scale=c.scale,
                                         kv_dtype=c.kv_dtype, max_context_len=c.max_context_len,
                                         k_scale=c.k_scale, v_scale=c.v_scale, out=self.out,
                                         workspace=self.ws, prepared=prepared)
        return self.pa.decode(self.q, self.kc, self.vc, self.tables, self.lens, block_size=c.bs,
                       scale=c.scale, kv_dtype=c.kv_dtype, max_context_len=c.max_context_len,
                       k_scale=c.k_scale, v_scale=c.v_scale, out=self.out, workspace=self.ws,
                       shared_frames=self.shared, prepared=prepared)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture each phase of the step in a HIP graph and replay the graphs "
                         "(default: launch every call from Python each step)")
    ap.add_argument("--mixed", action="store_true",
                    help="run the step's chunks and decodes in one pa_mixed_attention call "
                         "(workloads with both)")
    ap.add_argument("--mixed-mode", default="auto", choices=["auto", "split", "separate"],
                    help="launch mode of pa_mixed_attention (auto: the library's choice)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run three plain device copies of this many MiB before the timed steps "
                         "(a known-size reference for hardware byte counters)")
    ap.add_argument("--chunk-kv", default=None, choices=["bf16", "fp8"],
                    help="config 5 only: the same mixed step with this KV cache dtype (fp8: "
                         "per-tensor scales) -- the fp8 prefill-chunk variant")
    ap.add_argument("--chunk-block-size", type=int, default=None, choices=[16, 32],
                    help="config 5 only: the same mixed step with this block size")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="decode with pa_decode_shared: sequences whose tables begin with the same "
                         "frames (config 4's branches) read them once per group")
    ap.add_argument("--shared-run-max", type=int, default=None,
                    help="with --shared-prefix: at most this many sequences a run (default: as "
                         "many as a run's score columns hold)")
    ap.add_argument("--long", type=int, default=None, choices=[1, 4, 16],
                    help="long-context decode instead of a named config: this many sequences of "
                         "32,768 tokens at the 70B layer shape")
    ap.add_argument("--block-manager", action="store_true",
                    help="time the host block manager (no GPU): prompts, decode steps with their "
                         "block-table export, and copy-on-write forks, for the 70B-shape batch")
    args = ap.parse_args()
    if args.block_manager:
        block_manager_bench()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the library has no multi-GPU path and measures one GPU; --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_256_amd as pa
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    if args.long:
        case = workloads.long_context(args.long)
    elif args.chunk_kv or args.chunk_block_size:
        if args.config != 5:
            print("bench.py: --chunk-kv / --chunk-block-size apply to --config 5 only",
                  file=sys.stderr)
            sys.exit(2)
        case = workloads.config5_variant(kv_dtype=args.chunk_kv or "bf16",
                                         bs=args.chunk_block_size or 16)
    else:
        case = workloads.make(args.config)
    log(f"[bench] generated {case.name} in {time.time() - t0:.1f}s")
    st = DeviceState(case, dev)
    groups = None
    if args.shared_prefix:
        if not case.B:
            print("bench.py: --shared-prefix needs decodes", file=sys.stderr)
            sys.exit(2)
        groups = st.init_shared(dev, args.shared_run_max)
        log(f"[bench] {groups.num_runs} runs of sequences that share their first frames")
    torch.cuda.synchronize()
    log(f"[bench] caches filled on the GPU ({case.NB} frames)")

    flush = None if args.no_flush else torch.ones(128 << 20, dtype=torch.float32, device=dev)

    if args.calibration_copy_mib:
        src = torch.ones(args.calibration_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the three phases of a step; each is one call of the library
    if args.mixed:
        if case.chunk is None or not case.B:
            print("bench.py: --mixed needs a workload with chunks and decodes", file=sys.stderr)
            sys.exit(2)
        st.init_mixed(dev, args.mixed_mode)
        phases = [st.write, st.mixed, None]
    else:
        phases = [st.write, st.prefill if case.chunk is not None else None,
                  st.decode if case.B else None]
    if not args.graph:
        # every call's arguments are checked and marshalled once, before the timed loop: a step
        # then only issues the library calls, so no host work sits between the kernels
        phases = [f(prepared=True) if f is not None else None for f in phases]
    if args.graph:
        # one HIP graph per phase: a step replays the three graphs, so no host time sits
        # between the kernels of a phase
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for f in phases:
                if f is not None:
                    f()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for f in phases:
            if f is None:
                graphs.append(None)
                continue
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                f()
            graphs.append(gr)
        torch.cuda.synchronize()
        phases = [gr.replay if gr is not None else None for gr in graphs]

    def one_step(ev):
        ev[0].record()
        for i, f in enumerate(phases):
            if f is not None:
                f()
            ev[i + 1].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    warm = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for _ in range(args.warmup):
        if flush is not None:
            flush.sum()
        one_step(warm)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            flush.sum()
        one_step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
    write_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    chunk_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    dec_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    ms = float(step_ms.mean())

    kv_bytes = case.decode_kv_bytes() if case.B else 0
    qo_bytes = 2 * case.B * case.Hq * case.D * (4 if case.q_dtype == "f32" else 2)
    value = kv_bytes / (ms * 1e-3) / 1e9 if case.B else 0.0
    seqs_per_s = case.B / (ms * 1e-3)
    dec_avg = float(dec_ms.mean())
    achieved = kv_bytes / (dec_avg * 1e-3) / 1e9 if case.B and dec_avg > 0 else 0.0
    traffic = measured_traffic(case.name) if case.B else None
    kernels = ("decode_stream_kernel + decode_reduce_kernel" if case.B <= 1024 else
               "decode_plan_kernel + decode_stream_kernel + decode_reduce_kernel")
    if groups is not None:
        kernels = kernels + " (runs of sequences that share frames)"
        traffic = None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic[0] if traffic else None,
                "kernel": f"{kernels} (one {'pa_decode_shared' if groups is not None else 'pa_decode'} "
                          "call, timed with HIP events)",
                "avg_us": round(dec_avg * 1e3, 2),
                "algorithmic_bytes_per_launch": kv_bytes,
                "traffic_source": traffic[1] if traffic else None}
    extra = {"write_us": round(float(write_ms.mean()) * 1e3, 2),
             "decode_us": round(dec_avg * 1e3, 2),
             "decode_us_median": round(float(np.median(dec_ms)) * 1e3, 2),
             "decode_us_p10_p90": [round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                                   round(float(np.percentile(dec_ms, 90)) * 1e3, 2)],
             "wall_s_timed_loop": round(wall, 3), "flush_between_steps": flush is not None,
             "launch": "hip graph per phase" if args.graph else "eager, arguments marshalled once",
             "attention_calls": "pa_decode_shared" if groups is not None else
                                "pa_mixed_attention" if args.mixed else
                                "pa_prefill_chunk + pa_decode" if case.chunk is not None and case.B else
                                "pa_prefill_chunk" if case.chunk is not None else "pa_decode",
             "decode_shared_frames_hint": bool(case.B and st.shared)}
    if groups is not None:
        extra["shared_runs"] = groups.num_runs
        extra["shared_run_max"] = int(np.max(groups.run_size)) if len(groups.run_size) else 0
    if case.B and case.shares_frames:
        # frames several sequences reference are one copy in HBM: the bytes a decode that reads
        # each referenced frame once must move
        nblk = -(-case.context_lens.astype(np.int64) // case.bs)
        used = np.unique(np.concatenate([case.block_tables[b, :nblk[b]] for b in range(case.B)]))
        eb = {"f32": 4, "bf16": 2, "fp8": 1}[case.kv_dtype]
        extra["kv_unique_bytes_per_step"] = int(len(used)) * 2 * case.Hkv * case.bs * case.D * eb
        extra["kv_unique_gbs_decode"] = round(extra["kv_unique_bytes_per_step"] / (dec_avg * 1e-3) / 1e9, 1)
        # achieved / frac count every sequence's context (logical bytes, above the HBM rate when
        # shared frames come from the caches); the unique bytes are the least HBM traffic
        roofline["bytes"] = "logical (each sequence's context; shared frames counted per sequence)"
        roofline["unique_achieved"] = extra["kv_unique_gbs_decode"]
        roofline["unique_frac"] = round(extra["kv_unique_gbs_decode"] / HBM_PEAK_GBS, 4)
    if args.mixed:
        fl = chunk_flops(case)
        mavg = float(chunk_ms.mean())
        achieved = kv_bytes / (mavg * 1e-3) / 1e9
        extra.pop("decode_us")
        extra.pop("decode_us_p10_p90")
        extra["mixed_us"] = round(mavg * 1e3, 2)
        extra["mixed_us_p10_p90"] = [round(float(np.percentile(chunk_ms, 10)) * 1e3, 2),
                                     round(float(np.percentile(chunk_ms, 90)) * 1e3, 2)]
        extra["mixed_prefill_units"] = st.mixed_units
        extra["mixed_mode"] = args.mixed_mode
        extra["chunk_flop"] = fl
        extra["mixed_chunk_tflops"] = round(fl / (mavg * 1e-3) / 1e12, 2)
        extra["mixed_chunk_frac_of_mfma_bf16_peak"] = round(fl / (mavg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": "mixed_kernel + mixed_merge_kernel (one pa_mixed_attention call: "
                              "decode KV bytes over the whole launch, which also runs the chunk)",
                    "avg_us": extra["mixed_us"], "algorithmic_bytes_per_launch": kv_bytes,
                    "traffic_source": None}
        dec_avg = mavg
    elif case.chunk is not None:
        fl = chunk_flops(case)
        cavg = float(chunk_ms.mean())
        extra["chunk_us"] = round(cavg * 1e3, 2)
        extra["chunk_tflops"] = round(fl / (cavg * 1e-3) / 1e12, 2)
        extra["chunk_frac_of_mfma_bf16_peak"] = round(fl / (cavg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        extra["chunk_flop"] = fl
        if not case.B:
            roofline = {"bound": "mfma", "achieved": extra["chunk_tflops"],
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": extra["chunk_frac_of_mfma_bf16_peak"], "traffic": None,
                        "kernel": "prefill_chunk_kernel (+ reduce)", "avg_us": extra["chunk_us"]}
    log(f"[bench] step {ms * 1e3:.1f} us  decode {dec_avg * 1e3:.1f} us  -> {value:.0f} GB/s step, "
        f"{achieved:.0f} GB/s decode ({achieved / HBM_PEAK_GBS * 100:.1f}% of 8 TB/s)")

    cpu = None
    if not args.no_cpu_baseline and case.B:
        cpu = cpu_baseline(case, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "bf16 q / fp8-e4m3 kv"}[case.kv_dtype],
        "data": "synthetic (seeded, shapes of the named layer; no weights or datasets)",
        "config": {
            "workload": case.name,
            "cfg": case.meta.get("cfg", args.config),
            "batch": case.B,
            "q_heads": case.Hq, "kv_heads": case.Hkv, "head_dim": case.D,
            "block_size": case.bs, "kv_dtype": case.kv_dtype,
            "context_tokens": int(case.context_lens.sum()) if case.B else 0,
            "kv_bytes_per_step": kv_bytes,
            "q_out_bytes_per_step": qo_bytes,
            "seqs_per_s_per_layer": round(seqs_per_s, 1),
            "kv_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
            **extra,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def block_manager_bench():
    """Host-side rows of the path (the block manager): time the library's pa_bm_* calls on the
    70B-shape batch (256 sequences, prompts log-uniform in [128, 8192], 16-token blocks) and the
    plain-Python reference model on the same operations.  One JSON line."""
    import paged_kv_cache_256_amd as pa
    from oracle.block_manager import BlockManagerModel

    rng = np.random.default_rng(3)
    B, bs, steps = 256, 16, 200
    lens = np.clip(np.round(np.exp(rng.uniform(np.log(128), np.log(8192), B))), 128, 8192).astype(int)
    frames = int(sum(-(-(L + steps) // bs) for L in lens)) * 2 + 64
    prompts = [rng.integers(0, 32000, size=L).astype(np.int32) for L in lens]
    width = -(-(int(lens.max()) + steps) // bs)
    ids = np.arange(B, dtype=np.int64)

    def run(bm, n_steps, export):
        t0 = time.perf_counter()
        for b in range(B):
            bm.append_prompt(b, prompts[b])
        t1 = time.perf_counter()
        for _ in range(n_steps):
            bm.append(ids)
            if export:
                bm.block_tables(ids, width)
        t2 = time.perf_counter()
        return t1 - t0, (t2 - t1) / n_steps

    bm = pa.BlockManager(frames, bs)
    lib_prompt_s, lib_step_s = run(bm, steps, True)
    # copy-on-write: fork every sequence and append one token to each branch
    t0 = time.perf_counter()
    for b in range(B):
        bm.fork(b, B + b)
    _, pairs = bm.append(np.arange(B, 2 * B, dtype=np.int64))
    lib_fork_s = time.perf_counter() - t0
    bm.close()

    class ModelAdapter:
        def __init__(self):
            self.m = BlockManagerModel(frames, bs)

        def append_prompt(self, seq, toks):
            self.m.append_prompt(seq, toks)

        def append(self, seq_ids):
            self.m.append(seq_ids)

        def block_tables(self, seq_ids, w):
            return [self.m.block_table(int(s), w) for s in seq_ids]

    model_steps = 5
    model_prompt_s, model_step_s = run(ModelAdapter(), model_steps, True)
    tokens = int(lens.sum())
    line = {
        "metric": "host block manager: one decode step of 256 sequences (append + block-table export)",
        "value": round(lib_step_s * 1e6, 1), "unit": "us", "higher_is_better": False,
        "data": "synthetic (seeded prompt token ids)",
        "config": {"workload": "70B-shape batch: 256 sequences, prompts log-uniform in [128, 8192], bs 16",
                   "frames": frames, "prompt_tokens": tokens, "decode_steps": steps,
                   "prompts_us": round(lib_prompt_s * 1e6, 1),
                   "prompt_tokens_per_s": round(tokens / lib_prompt_s, 1),
                   "fork_and_cow_append_us": round(lib_fork_s * 1e6, 1),
                   "cow_copies": int(len(pairs))},
        "cpu_baseline": {"value": round(model_step_s * 1e6, 1), "unit": "us", "cores": 1,
                         "kind": "oracle",
                         "sample": f"the reference model on the same prompts and {model_steps} decode steps",
                         "prompts_us": round(model_prompt_s * 1e6, 1)},
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(case, budget_s: float):
    """The fp64 oracle (as it stands) on a bounded sample of the workload's sequences: the
    step's cache writes for those sequences and their decode.  Rate on the same KV-byte
    numerator as the GPU line."""
    import oracle
    from tests.gpu_harness import OracleStep

    t0 = time.time()
    o = OracleStep(case)
    log(f"[bench] oracle caches built in {time.time() - t0:.1f}s")
    rng = np.random.default_rng(0)
    order = rng.permutation(case.B)
    # calibrate on one sequence, then take as many as fit the budget
    probe = [int(order[0])]
    tp = time.perf_counter()
    o.decode(probe)
    per_token = (time.perf_counter() - tp) / max(1, int(case.context_lens[probe[0]]))
    pick, tokens = [], 0
    for b in order:
        L = int(case.context_lens[b])
        if pick and (tokens + L) * per_token > budget_s:
            break
        pick.append(int(b))
        tokens += L
    kw = dict(bs=case.bs, src_dtype=case.src_dtype, kv_dtype=case.kv_dtype,
              k_scale=case.k_scale, v_scale=case.v_scale)
    tstart = time.perf_counter()
    oracle.reshape_and_cache(o.kc, o.vc, case.new_k[pick], case.new_v[pick], case.new_slots[pick], **kw)
    o.decode(pick)
    dt = time.perf_counter() - tstart
    kv = case.decode_kv_bytes(np.array(pick))
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{len(pick)} of {case.B} sequences ({tokens} context tokens): their "
                      f"cache writes + fp64 decode, {dt:.1f}s",
            "seconds": round(dt, 2), "seqs_per_s": round(len(pick) / dt, 3),
            "host_cpu": cpu_model(), "host_logical_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
