"""Benchmark of the paged decode step on one MI355X.

A step is one pass of the whole hot path over one batch: append each
sequence's new token to the paged cache and decode attention of one query
token per sequence over its cache, in one launch (paged_decode_step).  The
headline workload is the Llama-8B-shaped batch: 64 sequences with context
lengths uniform in [128, 2048], 32 query / 8 KV heads, head_dim 128, block
size 16, bf16, blocks shuffled through an 8192-block pool.

The same JSON line then reports every other workload through the same
library calls: the tiny fp32 batch, the fp16 block-size sweep (16/32/64/128,
with its one-token append), the shared-prefix batch (sharing-unaware decode
and paged_attn_decode_shared), the long-context batch (128k to 1M tokens) and
four query tokens per sequence on the Llama-8B batch.

Inputs are resident in HBM before timing starts.  Steps rotate over several
copies of the pool where one copy would fit in the 256 MiB Infinity Cache, so
the bytes a step reads come from HBM.  Calls go to the C entry points with
their arguments marshalled once per input copy, so the timed region holds the
library's launches and not the Python binding's argument checks.

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
METRIC = "decode-attn KV-read GB/s and % of MI355X HBM peak; query tokens/s"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_cache_353_amd", "csrc")

# Sources the one-query decode kernel (the roofline kernel) is built and
# launched from: counter readings taken on another version of them are not
# reported.
STREAM_SOURCES = ["attn_decode.hip", "kv_write.hip", "pkv_device.h", "pkv_internal.h", "pkv_api.cpp"]


def say(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest() -> str:
    """Digest of the sources of the timed one-query decode kernel."""
    h = hashlib.sha256()
    paths = [os.path.join(CSRC, f) for f in STREAM_SOURCES] + [os.path.join(ROOT, "include", "pkv.h")]
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def build_workload(name: str, dev: str):
    from paged_kv_cache_353_amd import workloads as W
    if name == "llama8b":
        return W.llama8b_decode(dev)
    if name.startswith("sweep"):
        return W.block_size_sweep(int(name[len("sweep"):] or 16), dev)
    if name == "shared_prefix":
        return W.shared_prefix(dev)
    if name == "long_context":
        return W.long_context(dev)
    if name == "tiny":
        return W.tiny(dev)
    raise SystemExit(f"unknown workload {name!r}")


def replicas(inp, n: int):
    """n input sets with the same values at distinct HBM addresses."""
    from paged_kv_cache_353_amd.workloads import DecodeInputs
    sets = [inp]
    for _ in range(n - 1):
        sets.append(DecodeInputs(**{**inp.__dict__, "k_cache": inp.k_cache.clone(),
                                    "v_cache": inp.v_cache.clone()}))
    return sets


def traffic_for(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary of this workload (FETCH_SIZE and WRITE_SIZE, scaled by what the
    same counters read for a copy of known size), or None when there is none
    or it was taken on another version of the kernel sources."""
    path = os.path.join(PROFILES, f"attn_decode_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source") != source_digest():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parity_check(inp, out, pairs):
    """Sampled outputs of the timed data against the fp64 oracle (CPU)."""
    import numpy as np
    import oracle
    from paged_kv_cache_353_amd.workloads import to_numpy_bits
    q = to_numpy_bits(inp.q)
    kc = to_numpy_bits(inp.k_cache)
    vc = to_numpy_bits(inp.v_cache)
    want = oracle.paged_attn_decode(q, kc, vc, inp.block_tables.cpu().numpy(),
                                    inp.context_lens.cpu().numpy(), inp.block_size, inp.scale,
                                    inp.dtype, pairs=pairs)
    got = out.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for i, h in pairs:
        d = np.abs(got[i, h] - want[i, h])
        if not np.all(d <= 2e-3 + 1e-2 * np.abs(want[i, h])):
            raise SystemExit(f"parity check failed at seq {i} head {h}: max |d| {d.max():.3e}")
        worst = max(worst, float(np.linalg.norm(got[i, h] - want[i, h]) / np.linalg.norm(want[i, h])))
    return worst


# ---------------------------------------------------------------------------
# calls through the C entry points, arguments marshalled once per input copy
# ---------------------------------------------------------------------------

class Calls:
    """Pre-marshalled C calls of one workload: one argument tuple per input
    copy and call kind; each call checks the returned status."""

    def __init__(self, sets, outs, workspace, stream, max_context_len):
        from paged_kv_cache_353_amd import _lib
        self.lib = _lib.load_library()
        self.sets, self.outs = sets, outs
        ws, nws = workspace.data_ptr(), workspace.numel()
        st = stream.cuda_stream
        self.step_args, self.decode_args, self.write_args = [], [], []
        for s, o in zip(sets, outs):
            S, Hq, D = s.q.shape
            nb, Hkv, bs, _ = s.k_cache.shape
            mb = s.block_tables.shape[1]
            dt = _lib._dtype_code(s.q)
            self.step_args.append((o.data_ptr(), s.q.data_ptr(), s.k_new.data_ptr(), s.v_new.data_ptr(),
                                   s.k_cache.data_ptr(), s.v_cache.data_ptr(), s.block_tables.data_ptr(),
                                   s.context_lens.data_ptr(), S, Hq, Hkv, D, bs, mb, nb, max_context_len,
                                   s.scale, dt, ws, nws, st))
            self.decode_args.append((o.data_ptr(), s.q.data_ptr(), s.k_cache.data_ptr(), s.v_cache.data_ptr(),
                                     s.block_tables.data_ptr(), s.context_lens.data_ptr(), S, Hq, Hkv, D, bs,
                                     mb, nb, max_context_len, s.scale, dt, ws, nws, st))
            self.write_args.append((s.k_new.data_ptr(), s.v_new.data_ptr(), s.k_cache.data_ptr(),
                                    s.v_cache.data_ptr(), s.slot_mapping.data_ptr(), S, Hkv, D, bs, nb,
                                    Hkv * D, Hkv * D, dt, st))

    def _ok(self, status, what):
        if status != 0:
            raise RuntimeError(f"{what} failed: {self.lib.pkv_status_string(status).decode()}")

    def step(self, k):
        self._ok(self.lib.paged_decode_step(*self.step_args[k % len(self.step_args)]), "paged_decode_step")

    def decode(self, k):
        self._ok(self.lib.paged_attn_decode(*self.decode_args[k % len(self.decode_args)]), "paged_attn_decode")

    def write(self, k):
        self._ok(self.lib.paged_kv_write(*self.write_args[k % len(self.write_args)]), "paged_kv_write")

    def separate(self, k):
        self.write(k)
        self.decode(k)


def timed(fn, n, stream):
    """Average microseconds per call of fn(k), k = 0..n-1, back to back, with
    events on the stream the kernels run on."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for k in range(n):
        fn(k)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3


def warm_up(fn, n):
    """n untimed calls, then more until the GPU has been busy for about 0.2 s,
    so that timed calls do not run at the clocks of an idle GPU."""
    import torch
    for k in range(n):
        fn(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        for k in range(20):
            fn(k)
        torch.cuda.synchronize()


def per_call(fn, n, stream):
    """p10 / median / p90 of per-call durations (an event pair around each call)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for k in range(n):
        ev[k][0].record(stream)
        fn(k)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    each = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    pick = lambda f: round(each[min(len(each) - 1, int(f * (len(each) - 1) + 0.5))], 3)
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9), "calls": n}


def rates(nbytes, us, seqs, query_tokens=1):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 3), "kv_gbs": round(gbs, 2), "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
            "query_tokens_per_s": round(seqs * query_tokens / (us * 1e-6), 1)}


def setup(name, dev, nsets):
    """Workload, its input copies, outputs, a zeroed workspace and the calls."""
    import torch
    import paged_kv_cache_353_amd as pkv
    base = build_workload(name, dev)
    sets = replicas(base, nsets)
    S, Hq, Hkv, D = base.num_seqs, base.num_q_heads, base.num_kv_heads, base.head_dim
    maxL = base.max_context_len
    ws = torch.zeros(max(1, pkv.paged_attn_decode_workspace_size(S, Hq, Hkv, D, base.block_size, maxL)),
                     dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(s.q) for s in sets]
    calls = Calls(sets, outs, ws, torch.cuda.current_stream(), maxL)
    return base, sets, outs, ws, calls


def workload_line(name, dev, steps, warmup, nsets, stream):
    """Step, separate append + decode, decode alone and the append alone of
    one workload, each back to back over its input copies."""
    import torch
    base, sets, outs, ws, calls = setup(name, dev, nsets)
    warm_up(calls.step, max(2, warmup))
    step_us = timed(calls.step, steps, stream)
    sep_us = timed(calls.separate, steps, stream)
    dec_us = timed(calls.decode, steps, stream)
    wr_us = timed(calls.write, steps, stream)
    nbytes = base.kv_read_bytes()
    line = {"workload": base.name, "num_seqs": base.num_seqs, "block_size": base.block_size,
            "dtype": base.dtype, "context_tokens": int(base.lens.sum()), "kv_read_bytes_per_step": nbytes,
            "input_sets": nsets, "steps": steps, **rates(nbytes, step_us, base.num_seqs),
            "separate_write_then_decode_us": round(sep_us, 3), "decode_only_us": round(dec_us, 3),
            "kv_write_us": round(wr_us, 3)}
    del base, sets, outs, ws, calls
    torch.cuda.empty_cache()
    return line


# ---------------------------------------------------------------------------
# the CPU oracle on this host's cores
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_oracle(inp, budget_s: float, seqs=None, heads=None, with_append=True):
    """The fp64 oracle, as it stands, timed on this host over whole passes of
    a bounded sample of the workload (the append of the sample's tokens, then
    decode of the sampled sequences and query heads), repeated until about
    budget_s seconds.  Rates are per query token and per algorithmic KV byte
    of the sample, and the time of one whole step is extrapolated from them.
    The oracle's append copies the whole pool, so for multi-GiB pools the
    sample times the decode alone (with_append False)."""
    import numpy as np
    import oracle
    from paged_kv_cache_353_amd.workloads import to_numpy_bits
    S, Hq = inp.num_seqs, inp.num_q_heads
    seqs = list(range(S)) if seqs is None else list(seqs)
    heads = list(range(Hq)) if heads is None else list(heads)
    pairs = [(i, h) for i in seqs for h in heads]
    q = to_numpy_bits(inp.q)
    kc = to_numpy_bits(inp.k_cache)
    vc = to_numpy_bits(inp.v_cache)
    kn, vn = to_numpy_bits(inp.k_new), to_numpy_bits(inp.v_new)
    tables = inp.block_tables.cpu().numpy()
    lens = inp.context_lens.cpu().numpy()
    slots = inp.slot_mapping.cpu().numpy()
    sel = np.zeros(S, dtype=bool)
    sel[seqs] = True
    slots_s = np.where(sel, slots, -1)
    whole = len(seqs) == S and len(heads) == Hq
    passes, t_total = 0, 0.0
    while passes == 0 or t_total < budget_s:
        t0 = time.perf_counter()
        kc2, vc2 = oracle.paged_kv_write(kn, vn, kc, vc, slots_s) if with_append else (kc, vc)
        oracle.paged_attn_decode(q, kc2, vc2, tables, lens, inp.block_size, inp.scale, inp.dtype,
                                 pairs=None if whole else pairs)
        t_total += time.perf_counter() - t0
        passes += 1
    eb = 4 if inp.dtype == "f32" else 2
    sample_tokens = int(lens[seqs].sum())
    # a query token of the sample attends with len(heads) of its heads
    frac_heads = len(heads) / Hq
    sample_bytes = sample_tokens * inp.num_kv_heads * inp.head_dim * 2 * eb * frac_heads
    t_pass = t_total / passes
    all_bytes = int(lens.sum()) * inp.num_kv_heads * inp.head_dim * 2 * eb
    t_step = t_pass * all_bytes / max(sample_bytes, 1.0)
    return {"workload": inp.name,
            "sample": (f"{passes} pass(es) of {'append + ' if with_append else ''}decode over {len(seqs)} of {S} "
                       f"sequences x {len(heads)} of {Hq} query heads ({sample_tokens} context tokens) "
                       f"in {t_total:.1f} s"),
            "seconds_per_sample_pass": round(t_pass, 4), "step_seconds_extrapolated": round(t_step, 3),
            "query_tokens_per_s": round(S / t_step, 3),
            "kv_read_gbs": round(sample_bytes / t_pass / 1e9, 4)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b", help="headline workload (the others follow as extras)")
    ap.add_argument("--sets", type=int, default=4, help="rotating input copies (cold-cache timing)")
    ap.add_argument("--cpu-budget", type=float, default=4.0, help="seconds of CPU oracle timing per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="time the headline workload only")
    ap.add_argument("--no-long-context", action="store_true", help="skip the long-context extra")
    ap.add_argument("--query-tokens", type=int, default=4,
                    help="also time several query tokens per sequence (Llama-8B batch; 0 = skip)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus} GPUs, WORLD_SIZE={world}): "
              "the decode path is measured on a single MI355X; see the design notes for how "
              "it would shard.", file=sys.stderr)
        return 2

    import torch
    import paged_kv_cache_353_amd as pkv
    from paged_kv_cache_353_amd import _lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = "cuda:0"
    torch.cuda.set_device(0)
    pkv.load_library()
    stream = torch.cuda.current_stream()
    K, Wm = args.steps, args.warmup

    # ---- headline: the Llama-8B-shaped decode step
    say(f"building workload {args.workload}")
    nsets = max(1, args.sets if args.workload != "long_context" else 1)
    base, sets, outs, ws, calls = setup(args.workload, dev, nsets)
    S, Hq, Hkv, D = base.num_seqs, base.num_q_heads, base.num_kv_heads, base.head_dim
    maxL = base.max_context_len
    kv_bytes = base.kv_read_bytes()
    kv_unique = base.kv_unique_bytes()   # differs from kv_bytes only where blocks are shared

    # parity of the timed data, before timing (the step appends the same
    # bytes again on every later call, so the data stays the same)
    calls.step(0)
    torch.cuda.synchronize()
    worst = None
    if not args.no_parity:
        say("parity check on sampled outputs")
        pairs = [(i % S, (7 * i) % Hq) for i in range(0, S, max(1, S // 16))]
        worst = parity_check(sets[0], outs[0], pairs)

    # W untimed warmup steps, then more until the GPU has been busy for about
    # 0.2 s, so that the timed steps do not run at idle clocks
    warm_up(calls.step, Wm)
    w0 = time.perf_counter()
    step_us = timed(calls.step, K, stream)          # the timed region: K steps
    wall = time.perf_counter() - w0
    separate_us = timed(calls.separate, K, stream)  # context: the same work as two launches
    decode_only_us = timed(calls.decode, K, stream)
    step_spread = per_call(calls.step, min(K, 100), stream)
    # binding overhead, for context: the same step through the Python binding
    binding_us = timed(lambda k: pkv.paged_decode_step(
        outs[k % nsets], sets[k % nsets].q, sets[k % nsets].k_new, sets[k % nsets].v_new, sets[k % nsets].k_cache,
        sets[k % nsets].v_cache, sets[k % nsets].block_tables, sets[k % nsets].context_lens, base.block_size,
        base.scale, max_context_len=maxL, workspace=ws), K, stream)
    warm_us = timed(lambda k: calls.step(0), 20, stream)   # one copy, back to back: cache-warm context

    extras = {}
    if args.workload == "llama8b" and args.query_tokens > 0:
        # several query tokens per sequence (draft verification) on the same batch
        from paged_kv_cache_353_amd.workloads import multi_query
        T = args.query_tokens
        q4s = [multi_query(x, T, 353_019) for x in sets]
        o4s = [torch.empty_like(x) for x in q4s]
        mws = torch.zeros(max(1, pkv.paged_attn_decode_multi_workspace_size(S, T, Hq, Hkv, D)),
                          dtype=torch.uint8, device=dev)
        lib = calls.lib
        margs = [(o4.data_ptr(), q4.data_ptr(), x.k_cache.data_ptr(), x.v_cache.data_ptr(),
                  x.block_tables.data_ptr(), x.context_lens.data_ptr(), S, T, Hq, Hkv, D, base.block_size,
                  x.block_tables.shape[1], x.k_cache.shape[0], maxL, base.scale, _lib._dtype_code(x.q),
                  mws.data_ptr(), mws.numel(), stream.cuda_stream) for x, q4, o4 in zip(sets, q4s, o4s)]

        def multi_call(k):
            if lib.paged_attn_decode_multi(*margs[k % nsets]) != 0:
                raise RuntimeError("paged_attn_decode_multi failed")
        warm_up(multi_call, 3)
        multi_us = timed(multi_call, K, stream)
        extras["multi_query_decode"] = {
            "entry_point": f"paged_attn_decode_multi ({T} query tokens per sequence, causal)",
            **rates(kv_bytes, multi_us, S, T)}
        del q4s, o4s, mws

    head_name, head_seqs = base.name, S
    del sets, outs, ws, calls
    torch.cuda.empty_cache()

    if not args.no_extras and args.workload == "llama8b":
        ext = {}
        say("workload tiny")
        ext["tiny_fp32"] = workload_line("tiny", dev, K, Wm, 1, stream)
        for bs in (16, 32, 64, 128):
            say(f"workload sweep bs {bs}")
            ext[f"sweep_fp16_bs{bs}"] = workload_line(f"sweep{bs}", dev, max(10, K // 2), Wm, 2, stream)
        say("workload shared prefix")
        sp = workload_line("shared_prefix", dev, K, Wm, 4, stream)
        sp.update(shared_prefix_line(dev, K, stream))
        ext["shared_prefix_bf16"] = sp
        if not args.no_long_context:
            say("workload long context")
            ext["long_context_bf16"] = workload_line("long_context", dev, 10, 2, 1, stream)
        extras["workloads"] = ext

    value = kv_bytes / (step_us * 1e-6) / 1e9
    traffic = traffic_for(head_name)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(step_us * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": base.dtype,
        "data": "synthetic (seeded N(0,1) values, shuffled block tables; no dataset)",
        "config": {"workload": head_name, "num_seqs": S, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": base.block_size,
                   "context_tokens": int(base.lens.sum()), "max_context_len": maxL,
                   "kv_read_bytes_per_step": kv_bytes, "kv_unique_bytes_per_step": kv_unique,
                   "input_sets": nsets},
        "query_tokens_per_s": round(head_seqs / (step_us * 1e-6), 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "unique_kv_gbs": round(kv_unique / (step_us * 1e-6) / 1e9, 2),
        "step_launch_us": round(step_us, 3),
        "separate_write_then_decode_us": round(separate_us, 3),
        "decode_only_us": round(decode_only_us, 3),
        "python_binding_step_us": round(binding_us, 3),
        "warm_step_us": round(warm_us, 3),
        "step_us_per_call": step_spread,
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": "attn_stream_kernel (paged_decode_step: append + decode, one launch)",
                     "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic},
        "parity_worst_normwise": worst,
        **extras,
        "kernel_source": source_digest(),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baselines(dev, args.cpu_budget, args.no_extras or args.workload != "llama8b",
                                               args.workload)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


def shared_prefix_line(dev, steps, stream):
    """paged_attn_decode_shared on the forked batch: each group's prefix read
    once for all its members (group description derived on the host, untimed)."""
    import torch
    import paged_kv_cache_353_amd as pkv
    from paged_kv_cache_353_amd import _lib
    from paged_kv_cache_353_amd.sharing import shared_prefix_groups
    base = build_workload("shared_prefix", dev)
    sets = replicas(base, 4)
    S, Hq, Hkv, D = base.num_seqs, base.num_q_heads, base.num_kv_heads, base.head_dim
    maxL = base.max_context_len
    gs, pl = shared_prefix_groups(base.block_tables.cpu().numpy(), base.lens, base.block_size)
    gs_d = torch.from_numpy(gs).to(dev)
    pl_d = torch.from_numpy(pl).to(dev)
    sws = torch.zeros(max(1, pkv.paged_attn_decode_shared_workspace_size(S, len(gs) - 1, Hq, Hkv, D)),
                      dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(s.q) for s in sets]
    lib = _lib.load_library()
    sargs = [(o.data_ptr(), x.q.data_ptr(), x.k_cache.data_ptr(), x.v_cache.data_ptr(),
              x.block_tables.data_ptr(), x.context_lens.data_ptr(), gs_d.data_ptr(), pl_d.data_ptr(),
              S, len(gs) - 1, Hq, Hkv, D, base.block_size, x.block_tables.shape[1],
              x.k_cache.shape[0], maxL, base.scale, _lib._dtype_code(x.q), sws.data_ptr(), sws.numel(),
              stream.cuda_stream) for x, o in zip(sets, outs)]

    def shared_call(k):
        if lib.paged_attn_decode_shared(*sargs[k % 4]) != 0:
            raise RuntimeError("paged_attn_decode_shared failed")
    warm_up(shared_call, 3)
    us = timed(shared_call, steps, stream)
    nbytes, unique = base.kv_read_bytes(), base.kv_unique_bytes()
    line = {"shared_decode": {
        "entry_point": "paged_attn_decode_shared (each group's prefix streamed once for all its members)",
        "groups": len(gs) - 1, "shared_tokens_per_group": int(pl[0]), "us": round(us, 3),
        "unique_kv_bytes": unique, "unique_kv_gbs": round(unique / (us * 1e-6) / 1e9, 2),
        "unique_pct_of_hbm_peak": round(100.0 * unique / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
        "logical_kv_gbs": round(nbytes / (us * 1e-6) / 1e9, 2),
        "query_tokens_per_s": round(S / (us * 1e-6), 1)}}
    del base, sets, outs, sws
    torch.cuda.empty_cache()
    return line


def cpu_baselines(dev, budget, headline_only, headline):
    """The oracle on this host's cores: the headline workload first, then the
    others on bounded samples; one entry per workload."""
    import torch
    say("timing the CPU oracle on bounded samples")
    cores = len(os.sched_getaffinity(0))
    entries = {}
    plan = [(headline, None, None, True)]
    if not headline_only:
        plan += [("tiny", None, None, True),
                 ("sweep16", range(0, 128, 16), None, False),       # 8 of 128 sequences, all heads
                 ("shared_prefix", range(0, 128, 16), None, True),  # one sample of each of 8 prompts
                 ("long_context", [0], range(0, 32, 8), False)]      # the 128k sequence, 4 of 32 heads
    for name, seqs, heads, app in plan:
        inp = build_workload(name, dev)
        entries[inp.name] = cpu_oracle(inp, budget, seqs, heads, app)
        del inp
        torch.cuda.empty_cache()
    head = next(iter(entries.values()))
    return {"value": head["query_tokens_per_s"], "unit": "query tokens/s", "cores": cores, "kind": "oracle",
            "sample": head["sample"], "cpu_model": cpu_model(), "blas_threads": blas_threads(),
            "kv_read_gbs": head["kv_read_gbs"], "per_workload": entries}


if __name__ == "__main__":
    sys.exit(main())
