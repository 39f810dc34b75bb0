"""Benchmark of one decode step of the rotated-codec KV cache on one MI355X.

A step is the whole hot path for one new token per sequence: append it (encode
K and V rows: rotate, norm, nearest centroid, pack), rotate q, split-K decode over
all visible tokens, LSE merge, inverse-rotate the output.  --path picks the calls:
  step      tq_decode_step: two kernels; the token is appended by extra work
            groups of the decode kernel while the splits stream the older tokens
            (default);
  fused     tq_encode_append -> tq_decode_attention_fused (three kernels);
  separate  tq_encode_append -> tq_rotate_q -> tq_decode_attention ->
            tq_inverse_rotate_out (five kernels);
  chunk     tq_encode_append of the last --q-len tokens -> tq_decode_chunk_fused
            (--q-len query positions per head, causal within the chunk).
--v-skip-threshold turns on sparse V; --q-scale multiplies the queries (peaked
weights, where sparse V has tiles to skip).
Inputs are seeded synthetic ones of the Qwen2.5-7B-shaped layer (B=1, Hq=28,
Hkv=4, head dim 128, 8192 visible tokens, turbo3 K and V) unless --workload says
otherwise.  The cache is replicated into distinct HBM copies (>= 1 GiB in all)
and the steps rotate through them, so every step streams its cache from HBM
rather than from the 256 MB Infinity Cache (each copy stands for another layer
of the model); the timed steps use copies the warm-up did not touch, after a
512 MiB copy has flushed the Infinity Cache.  Steps are captured in HIP graphs
(uploaded before the warm-up) and replayed, so host launch overhead is not in
the timed region: exactly --warmup untimed steps, then exactly --steps timed ones.

Prints ONE JSON line.  value = KV token-heads per second of whole steps
(visible tokens x KV heads / step time).  roofline = the decode call
(split-K kernel + LSE combine) timed by HIP events on its stream around a run of
calls enqueued eagerly behind a GPU sleep, so they run back to back: algorithmic
packed K+V bytes per call / average call duration (both kernels of the call),
against 8 TB/s.  With the defaults the line also carries "per_workload": the
same call timing and parity for the 16K fp16-K + turbo4-V layer, the batched
turbo4 workload and the ragged turbo3 workload (measured after the timed steps).
cpu_baseline = the float64 oracle (oracle/) doing the same step over a process
pool on the host cores (one worker per (sequence, KV head, token block) unit,
one BLAS thread each); its output for sequence 0 also gates the run: the GPU's
output of the timed step must sit within the tests' parity bars (rel-L2 1e-3,
max-abs 5e-3) and its codes must equal the oracle's outside the 1e-5 boundary
margin, reported as "parity", or bench.py exits non-zero.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized-KV decode attention: KV tokens/s/head + % of HBM roofline"
HBM_PEAK_GBS = 8000.0
BYTES_PER_TOKEN_HEAD = {"turbo3": 50, "turbo4": 66, "f16": 256}
EXTRA_WORKLOADS = (2, 3, 4)     # carried in the default line besides the headline workload
CODE_SLICE_TOKENS = 4096         # tokens of sequence 0 whose codes the parity record compares


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3200)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--workload", type=int, default=1, help="workload index (0..4); default the 8K Qwen2.5-7B layer")
    p.add_argument("--path", choices=("step", "fused", "separate", "chunk"), default="step",
                   help="calls per step (see the module docstring)")
    p.add_argument("--variant", type=int, default=0,
                   help="decode kernel variant of --path separate (0 default = MFMA, 1 VALU reference)")
    p.add_argument("--copies-gib", type=float, default=1.0, help="total size of the rotated cache copies")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--extra-cpu-seconds", type=float, default=5.0,
                   help="budget of the oracle's timing on each of the other workloads (0 skips it)")
    p.add_argument("--no-extra", action="store_true", help="skip the per-workload records of the other workloads")
    p.add_argument("--v-skip-threshold", type=float, default=0.0,
                   help="sparse-V weight threshold of the decode calls (0 = exact attention)")
    p.add_argument("--k-skip-threshold", type=float, default=0.0,
                   help="sparse-K weight threshold of the decode calls (0 = exact attention)")
    p.add_argument("--formats", default=None,
                   help="K/V formats instead of the workload's, e.g. f16/f16 (the uncompressed comparison cache)")
    p.add_argument("--q-len", type=int, default=4,
                   help="query positions per sequence of --path chunk (a causal chunk of the last tokens)")
    p.add_argument("--q-scale", type=float, default=1.0,
                   help="multiply the synthetic queries (e.g. 16 for peaked attention weights)")
    return p.parse_args(argv)


KERNEL_SOURCES = tuple("quantized_kv_cache_decode_amd/csrc/" + f
                       for f in ("api.hip", "decode_mfma.hip", "decode_ref.hip", "combine.hip", "tq_device.h",
                                 "tq_encode.h", "tq_launch.h"))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash():
    """sha256 of the decode and merge kernel sources and of the split planner (ties recorded
    counters to the code)."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload_name):
    """HBM bytes per decode call from the committed FETCH_SIZE/WRITE_SIZE profile, or None
    when there is none for this workload or the kernels changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    rec = t.get("workloads", {}).get(workload_name)
    return None if rec is None else rec["bytes_per_call"]


def algorithmic_bytes(w, lengths):
    return int(sum(lengths)) * w.num_kv_heads * (BYTES_PER_TOKEN_HEAD[w.k_format] + BYTES_PER_TOKEN_HEAD[w.v_format])


def clone_cache(master):
    """A new Cache whose device buffers are copies of master's (distinct HBM)."""
    import copy

    import quantized_kv_cache_decode_amd as tq
    c = copy.copy(master)
    for name in ("k_data", "k_norms", "v_data", "v_norms", "seq_lens"):
        t = getattr(master, name)
        setattr(c, name, None if t is None else t.clone())
    c.lengths = master.lengths.copy()
    c._desc = tq.binding.tq_cache(
        master.batch, master.num_kv_heads, 128, master.capacity, master._desc.k_format, master._desc.v_format,
        c.k_data.data_ptr(), 0 if c.k_norms is None else c.k_norms.data_ptr(), c.v_data.data_ptr(),
        0 if c.v_norms is None else c.v_norms.data_ptr(), c.seq_lens.data_ptr(), master.k_signs.data_ptr(),
        master.v_signs.data_ptr(),
        master.k_codebook.data_ptr(), master.v_codebook.data_ptr(), master._desc.v_skip_threshold,
        master._desc.k_skip_threshold)
    return c


def cache_bytes(c):
    return sum(t.numel() * t.element_size() for t in (c.k_data, c.k_norms, c.v_data, c.v_norms) if t is not None)


# ============================================================================ oracle leg
# Everything below that imports oracle/ is the CPU baseline and the parity gate; the GPU
# path above and in main() never calls it.

def _oracle_unit(task, barrier, results):
    """One worker of the CPU baseline: the oracle's share of a decode step for one
    (sequence b, KV head h, token block [t0, t1)) unit, repeated until the budget is spent.

    Per repetition: encode the appended token when the block holds slot L-1, dequantise the
    block's K and V rows (float64, original basis) and form the unnormalised partial (m, l, o)
    of the G query heads of h over them.  BLAS runs single-threaded in every worker."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    from dataclasses import replace

    from oracle import attention as att
    from oracle import codec, reference
    from synth import get_workload, kv_slice, new_token_kv, queries, sign_vector
    from tests.conftest import load_codebook
    uid, widx, formats, seed, b, h, t0, t1, L, budget = task
    w = get_workload(widx)
    if formats:
        w = replace(w, k_format=formats[0], v_format=formats[1])
    cbs = {"turbo3": load_codebook("turbo3"), "turbo4": load_codebook("turbo4")}
    sk, sv = sign_vector(seed, "k"), sign_vector(seed, "v")
    pre = L - 1                       # the step appends token L-1
    k16 = kv_slice(w, seed, "k", b, h, pre)[None, t0:min(t1, pre)]
    v16 = kv_slice(w, seed, "v", b, h, pre)[None, t0:min(t1, pre)]
    holds_new = t1 == L
    if holds_new:                     # the appended row's slot, filled by the timed loop
        k16 = np.concatenate([k16, np.zeros((1, 1, 128), np.float16)], axis=1)
        v16 = np.concatenate([v16, np.zeros((1, 1, 128), np.float16)], axis=1)
    enc = reference.encode_sequence(k16, v16, w.k_format, w.v_format, sk, sv, cbs)
    kn = new_token_kv(w, seed, "k", b, h, 0)[None]
    vn = new_token_kv(w, seed, "v", b, h, 0)[None]
    G = w.group
    q_rows = np.asarray(queries(w, seed)[b][h * G:(h + 1) * G], dtype=np.float64)
    n_tok = t1 - t0
    barrier.wait()
    start = time.perf_counter()
    reps = 0
    while True:
        if holds_new:
            s = n_tok - 1
            if w.k_format == "f16":
                enc["k_f16"][:, s] = kn[:, 0]
            else:
                c, n = codec.encode(kn, sk, cbs[w.k_format])
                enc["k_codes"][:, s], enc["k_norms"][:, s] = c[:, 0], n[:, 0]
            if w.v_format == "f16":
                enc["v_f16"][:, s] = vn[:, 0]
            else:
                c, n = codec.encode(vn, sv, cbs[w.v_format])
                enc["v_codes"][:, s], enc["v_norms"][:, s] = c[:, 0], n[:, 0]
        k_hat, v_hat = reference.dequant_sequence(enc, w.k_format, w.v_format, sk, sv, cbs, n_tok)
        part = att.partial(q_rows, k_hat[0], v_hat[0], reference.SCALE)
        reps += 1
        el = time.perf_counter() - start
        if el >= budget:
            break
    results.put((uid, reps, el, n_tok, part))


def cpu_baseline(w, widx, formats, seed, budget_s):
    """The float64 oracle doing the step for sequence 0 (append one token + full-dequant
    attention over all its visible tokens) over a process pool on the host cores.

    Units are (sequence 0, KV head, token block): the KV heads, each cut into enough token
    blocks that there is one unit per available core.  Every worker sets up its unit (not
    timed), waits at a barrier, then repeats its unit for the budget; the rate is the sum of
    the workers' rates.  Returns (record, o): o is the oracle's float64 output [Hq, 128] of
    sequence 0 for the step, the LSE merge of the units' last partials."""
    import multiprocessing as mp
    import queue

    from oracle import attention as att
    from synth.gen import context_lengths
    host_cores = len(os.sched_getaffinity(0))
    b = 0
    L = int(context_lengths(w, seed)[b])
    H = w.num_kv_heads
    blocks = max(1, min(host_cores // H, L // 64))
    bounds = [(L * i) // blocks for i in range(blocks + 1)]
    tasks = [(h * blocks + i, widx, formats, seed, b, h, bounds[i], bounds[i + 1], L, budget_s)
             for h in range(H) for i in range(blocks)]
    ctx = mp.get_context("spawn")     # fresh interpreters: the parent holds a GPU context
    barrier, results = ctx.Barrier(len(tasks)), ctx.Queue()
    wall0 = time.perf_counter()
    procs = [ctx.Process(target=_oracle_unit, args=(t, barrier, results), daemon=True) for t in tasks]
    for p in procs:
        p.start()
    got, deadline = [], time.time() + 600 + 4 * budget_s
    while len(got) < len(procs):
        try:
            got.append(results.get(timeout=1.0))
        except queue.Empty:
            dead = [p.exitcode for p in procs if p.exitcode not in (None, 0)]
            if dead or time.time() > deadline:
                for p in procs:
                    p.terminate()
                raise RuntimeError(f"CPU baseline workers failed (exit codes {dead}) or timed out")
    for p in procs:
        p.join(timeout=60)
    wall_s = time.perf_counter() - wall0
    got.sort(key=lambda r: r[0])
    rate = sum(r[1] * r[3] / r[2] for r in got)        # token-heads per second (one KV head per unit)
    o = np.concatenate([att.combine([got[h * blocks + i][4] for i in range(blocks)]) for h in range(H)])
    reps = [r[1] for r in got]
    rec = {
        "value": rate,
        "unit": "KV token-heads/s",
        "cores": len(procs),
        "host_cores": host_cores,
        "kind": "oracle",
        "wall_s": wall_s,          # the pool's whole run: start-up, unit set-up, the timed repetitions
        "sample": f"sequence 0 of {w.name}: append 1 token + float64 full-dequant attention over {L} tokens x "
                  f"{H} KV heads x {w.group} query heads each, as {len(procs)} single-threaded worker processes "
                  f"(one per (KV head, token block) unit, {blocks} blocks per head), {budget_s:.0f} s each, "
                  f"{min(reps)}-{max(reps)} repetitions per unit",
    }
    return rec, o


def oracle_parity(cache, w, b, L_b, k16, v16, q_b, got_b, o_ref=None, codebooks=None):
    """Parity of one sequence of the timed step's output: against o_ref (the oracle's end-to-end
    output, when given) or the oracle on the GPU-written bytes; codes and norms of the first
    CODE_SLICE_TOKENS tokens against the oracle's encode of the same rows."""
    from tests import support as S
    from tests.conftest import load_codebook
    codebooks = codebooks or {"turbo3": load_codebook("turbo3"), "turbo4": load_codebook("turbo4")}
    if o_ref is None:
        o_ref = S.oracle_on_bytes(cache, b, L_b, q_b, codebooks)
        against = "oracle on the GPU-written bytes"
    else:
        against = "oracle end to end (its own encode)"
    rel, mx = S.errors(got_b, o_ref)
    n = L_b if w.v_format == "f16" else min(L_b, CODE_SLICE_TOKENS)   # (fp16 rows: no encode, all of them)
    codes = {"tokens": n}
    try:
        m, g, t = S.compare_codes(cache, b, k16[:, :n], v16[:, :n], n, w, codebooks)
        codes.update(mismatches=m, within_margin=g, total=t, ok=bool(m <= g <= 1e-4 * max(t, 1)))
    except AssertionError as e:       # norms differ, or codes differ outside the margin
        codes.update(ok=False, error=str(e).splitlines()[0][:200])
    return {"sequence": b, "against": against, "rel_l2": rel, "max_abs": mx, "rel_l2_bound": 1e-3,
            "max_abs_bound": 5e-3, "codes": codes,
            "ok": bool(rel <= 1e-3 and mx <= 5e-3 and codes["ok"])}


# ============================================================================ GPU timing

def hip_graph_upload(graph):
    """Upload an instantiated graph to the device (hipGraphUpload) so that its first replay
    does not carry the upload; best effort (a no-op where the handle is not exposed)."""
    import ctypes

    import torch
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")      # the runtime torch already loaded
        hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        ex = graph.raw_cuda_graph_exec()
        return hip.hipGraphUpload(ctypes.c_void_p(int(ex)), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    except Exception:  # pragma: no cover
        return False


def time_calls(call, caches, n_calls, with_host=False):
    """Average duration (ms) of n_calls back-to-back calls, one HIP event pair on the launch
    stream around them all.  Events cannot be recorded inside a captured graph here, so the
    calls are enqueued eagerly behind a GPU sleep; the sleep is checked to outlast the host's
    enqueueing (else the GPU would wait for the host between calls and the figure would be the
    host's), and lengthened until it does.  with_host: also the host's enqueueing time per
    call (ms)."""
    import torch
    cycles = int(1e8)
    for _ in range(4):
        es, e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        es.record()
        torch.cuda._sleep(cycles)
        e0.record()
        h0 = time.perf_counter()
        for i in range(n_calls):
            call(caches[i % len(caches)])
        host_ms = (time.perf_counter() - h0) * 1e3
        e1.record()
        torch.cuda.synchronize()
        if es.elapsed_time(e0) > 1.2 * host_ms:
            ms = e0.elapsed_time(e1) / n_calls
            return (ms, host_ms / n_calls) if with_host else ms
        cycles *= 4
    raise RuntimeError(f"the GPU sleep never outlasted the host's enqueueing of {n_calls} calls ({host_ms:.1f} ms)")


STEADY_WARM_S = 0.6      # load before the steady-state window: the engine clock settles within ~0.5 s
STEADY_WINDOW_S = 0.1


def call_time(call, caches, n_burst):
    """Average duration (ms) of one call under load, and how it was taken.

    A burst of n_burst calls behind a GPU sleep starts from an idle chip, and the chip's power
    management then lowers the engine clock over the next few hundred ms (2.4 GHz idle, ~2.08
    GHz under a sustained decode load), undershooting on the way: on the batched turbo4
    workload bursts of 2-8 calls and a continuous run both give ~181 us per call, bursts of
    16-192 calls 204-229 us.  So where the host stays well ahead of the GPU (its enqueueing
    under half the call time), calls are enqueued continuously, STEADY_WARM_S seconds of them
    untimed, and one HIP event pair brackets the next STEADY_WINDOW_S seconds: the steady
    state a serving loop runs in.  Short calls, which the host cannot stay ahead of and which
    load the chip lightly, keep the burst figure."""
    import torch
    burst_ms, host_ms = time_calls(call, caches, n_burst, with_host=True)
    if host_ms >= 0.5 * burst_ms:
        return burst_ms, {"call_timing": f"burst of {n_burst} calls behind a GPU sleep"}
    n_warm = int(math.ceil(STEADY_WARM_S * 1e3 / burst_ms))
    n_win = max(64, int(math.ceil(STEADY_WINDOW_S * 1e3 / burst_ms)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(n_warm):
        call(caches[i % len(caches)])
    e0.record()
    for i in range(n_win):
        call(caches[(n_warm + i) % len(caches)])
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n_win, {
        "call_timing": f"steady state: {n_win} calls after {n_warm} untimed ({STEADY_WARM_S} s of load)",
        "call_us_burst": burst_ms * 1e3, "host_enqueue_us": host_ms * 1e3}


def single_call_us(call, caches, n_calls=21):
    """Latency of one call on its own: the GPU idle before it (synchronised), one HIP event pair
    around it, a different cache copy each time; the median over n_calls (µs).  The events add
    about 2 µs on calls this short."""
    import torch
    ts = []
    for i in range(n_calls):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call(caches[(i + 1) % len(caches)])
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(ts))


def calls_to_time(n_copies):
    """Back-to-back calls in one event-timed run: at least 8, at most 192 (more would fill the
    launch queue while the GPU sleeps, and the host would wait for the GPU), and no more than
    the copies where there are enough (a copy comes back only after >= 1 GiB of other copies)."""
    return max(8, min(192, 64 * n_copies))


def flush_infinity_cache():
    """Write and read 512 MiB of other memory, so cache copies touched before are out of the
    256 MB Infinity Cache."""
    import torch
    a = torch.empty(1 << 27, dtype=torch.float32, device="cuda")
    a.fill_(1.0)
    b = a.clone()
    del a, b


def stream_read_ceiling(gib=1.0):
    """The practical HBM read ceiling on this GPU: the library's plain streaming-read kernel
    (tq_stream_read) over a 1 GiB buffer at several grid sizes, 10 timed passes each; the
    best rate in GB/s."""
    import torch

    import quantized_kv_cache_decode_amd as tq
    n = int(gib * (1 << 30)) // 16 * 16
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    best = (0.0, 0)
    for blocks in (8192, 32768, 131072):
        sums = torch.zeros(blocks, dtype=torch.int32, device="cuda")
        for _ in range(2):
            tq.tq_stream_read(src, sums)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            tq.tq_stream_read(src, sums)
        e1.record()
        torch.cuda.synchronize()
        gbs = n / (e0.elapsed_time(e1) / 10) / 1e6
        best = max(best, (gbs, blocks))
    del src
    torch.cuda.empty_cache()
    return {"kernel": "stream_read_kernel (tq_stream_read)", "bytes": n, "best_blocks": best[1],
            "achieved": best[0], "unit": "GB/s", "frac_of_peak": best[0] / HBM_PEAK_GBS}


def setup_copies(w, seed, copies_gib, min_copies=1):
    """Prefill L-1 tokens of every sequence (setup) and replicate the cache into distinct HBM
    copies of >= copies_gib in all."""
    from tests import support as S
    master, k_list, v_list, L, q_np = S.prefill_and_step(w, seed)
    per_copy = cache_bytes(master)
    n_copies = max(min_copies, int(math.ceil(copies_gib * (1 << 30) / per_copy)))
    caches = [master] + [clone_cache(master) for _ in range(n_copies - 1)]
    return caches, k_list, v_list, L, q_np


def extra_workload(widx, seed, with_oracle, codebooks, ceiling_gbs, cpu_seconds):
    """Call timing and parity of tq_decode_step on another workload (not the timed steps), and
    the oracle's rate on the same workload (cpu_seconds of host time; 0 skips it)."""
    import torch

    import quantized_kv_cache_decode_amd as tq
    from synth import get_workload
    from tests import support as S
    w = get_workload(widx)
    caches, k_list, v_list, L, q_np = setup_copies(w, seed, 1.0, min_copies=2)
    pre = (L - 1).astype(np.int32)
    kn, vn = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in S.new_token_rows(w, seed))
    q = torch.from_numpy(np.ascontiguousarray(q_np)).cuda()
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float16, device="cuda")
    ws = torch.zeros(tq.tq_decode_workspace_size(caches[0], w.num_q_heads, pre), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(128.0)

    def call(c):
        tq.tq_decode_step(c, kn, vn, q, scale, out, ws, seq_lens_host=pre)

    call(caches[0])
    torch.cuda.synchronize()
    n_calls = calls_to_time(len(caches))
    flush_infinity_cache()
    call_ms, how = call_time(call, caches, n_calls)
    alg = algorithmic_bytes(w, L)
    achieved = alg / (call_ms * 1e-3) / 1e9
    th = int(L.sum()) * w.num_kv_heads
    rec = {"call_us": call_ms * 1e3, **how, "cache_copies": len(caches),
           "single_call_us": single_call_us(call, caches),
           "algorithmic_bytes_per_call": alg, "achieved_GBs": achieved, "frac": achieved / HBM_PEAK_GBS,
           "frac_of_read_ceiling": achieved / ceiling_gbs,
           "kv_token_heads_per_s": th / (call_ms * 1e-3),
           "q_token_heads_per_s": th * w.group / (call_ms * 1e-3),
           "traffic": recorded_traffic(w.name), "parity": None, "cpu_baseline": None}
    if with_oracle:
        got = out.cpu().numpy()
        rec["parity"] = oracle_parity(caches[0], w, 0, int(L[0]), k_list[0], v_list[0], q_np[0], got[0],
                                      codebooks=codebooks)
        if cpu_seconds > 0:
            rec["cpu_baseline"], _ = cpu_baseline(w, widx, None, seed, cpu_seconds)
    del caches, k_list, v_list, kn, vn, q, out, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return w.name, rec


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the decode path is built and measured "
              "on a single MI355X; sharding is described, not built.", file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_kv_cache_decode_amd as tq
    from synth import get_workload, queries
    from tests import support as S
    tq.load_library()
    torch.cuda.set_device(0)
    w = get_workload(args.workload)
    formats = None
    if args.formats:
        from dataclasses import replace
        formats = tuple(args.formats.split("/"))
        w = replace(w, k_format=formats[0], v_format=formats[1])
    seed = 0
    K, W = int(args.steps), int(args.warmup)
    if K < 1 or W < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")

    # ---- setup (not timed): prefill L-1 tokens, replicate the cache into distinct copies
    caches, k_list, v_list, L, q_np = setup_copies(w, seed, args.copies_gib)
    for c in caches:
        c.v_skip_threshold = args.v_skip_threshold
        c.k_skip_threshold = args.k_skip_threshold
    n_copies = len(caches)
    master = caches[0]
    pre = (L - 1).astype(np.int32)
    kn, vn = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in S.new_token_rows(w, seed))
    q_np = (q_np.astype(np.float32) * args.q_scale).astype(q_np.dtype)
    q = torch.from_numpy(np.ascontiguousarray(q_np)).cuda()
    B, Hq = w.batch, w.num_q_heads
    q_rot = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    out_rot = torch.empty_like(q_rot)
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    ws = torch.zeros(max(tq.tq_decode_workspace_size(master, Hq, L), tq.tq_decode_workspace_size(master, Hq, pre)),
                     dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(128.0)
    if args.path == "chunk":
        # the chunk: the last q_len tokens of every sequence, re-appended each step, and
        # q_len query positions per head attending causally
        Tq = args.q_len
        chunk_pre = (L - Tq).astype(np.int32)
        kc = S.padded_tensor([k[:, int(L[b]) - Tq:int(L[b])] for b, k in enumerate(k_list)], Tq)
        vc = S.padded_tensor([v[:, int(L[b]) - Tq:int(L[b])] for b, v in enumerate(v_list)], Tq)
        qc_np = np.stack([queries(w, seed, step=t) for t in range(Tq)], axis=2)
        qc = torch.from_numpy(np.ascontiguousarray((qc_np.astype(np.float32) * args.q_scale).astype(qc_np.dtype))).cuda()
        out_c = torch.empty((B, Hq, Tq, 128), dtype=torch.float16, device="cuda")
        ws = torch.zeros(tq.tq_decode_workspace_size(master, Hq * Tq, L), dtype=torch.uint8, device="cuda")
    # a plain 512 MiB device copy (setup, untimed): its FETCH_SIZE / WRITE_SIZE counters
    # calibrate the HBM traffic figures read for the decode kernel in the same profile
    calib = torch.empty(1 << 27, dtype=torch.float32, device="cuda")
    calib.copy_(torch.ones_like(calib))
    del calib

    if args.variant and args.path != "separate":
        sys.exit("--variant applies to --path separate only")
    sep = args.path == "separate"

    def decode_call(c):
        """The timed call: append + decode for the step path, decode alone otherwise."""
        if args.path == "step":
            tq.tq_decode_step(c, kn, vn, q, scale, out, ws, seq_lens_host=pre)
        elif args.path == "chunk":
            tq.tq_decode_chunk_fused(c, qc, scale, out_c, ws, seq_lens_host=L)
        elif sep:
            tq.tq_decode_attention(c, q_rot, scale, out_rot, ws, seq_lens_host=L, variant=args.variant)
        else:
            tq.tq_decode_attention_fused(c, q, scale, out, ws, seq_lens_host=L)

    def step(i):
        # Every step writes the same token into slot L-1 of its cache copy and attends over
        # L tokens, so replays are idempotent and the copies keep their length.
        c = caches[i % n_copies]
        if args.path == "chunk":
            tq.tq_encode_append(c, kc, vc, seq_lens_host=chunk_pre)
        elif args.path != "step":
            tq.tq_encode_append(c, kn, vn, seq_lens_host=pre)
        if sep:
            tq.tq_rotate_q(c, q, q_rot)
        decode_call(c)
        if sep:
            tq.tq_inverse_rotate_out(c, out_rot, out)

    # Warm-up steps use copies 0, 1, ...; the timed steps continue the rotation from copy W,
    # so with --steps + --warmup <= the number of copies no timed step finds its copy in a cache.
    warm_idx = [i % n_copies for i in range(W)]
    timed_idx = [(W + i) % n_copies for i in range(K)]
    step(0)                           # load the kernels' code objects before any capture (setup)
    torch.cuda.synchronize()

    def plan(idx):
        """Graphs for a list of step indices: (graph over the first min(len, n_copies) steps,
        replays) + (graph over the remainder, 1); the rotation is periodic in n_copies."""
        n = len(idx)
        if n == 0:
            return []
        full = min(n, n_copies)
        parts = [(idx[:full], n // full)]
        if n % full:
            parts.append((idx[:n % full], 1))
        return parts

    use_graph = not args.no_graph
    graphs = {}
    if use_graph:
        try:
            for name, idx in (("warm", warm_idx), ("timed", timed_idx)):
                graphs[name] = []
                for sub, reps in plan(idx):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        for i in sub:
                            step(i)
                    hip_graph_upload(g)
                    graphs[name].append((g, reps))
        except Exception as e:  # pragma: no cover - reported, then eager timing
            print(f"graph capture unavailable ({e!r}); timing eager launches", file=sys.stderr)
            graphs, use_graph = {}, False

    def run(name, idx):
        if use_graph:
            for g, reps in graphs[name]:
                for _ in range(reps):
                    g.replay()
        else:
            for i in idx:
                step(i)

    run("warm", warm_idx)
    torch.cuda.synchronize()
    flush_infinity_cache()
    torch.cuda.synchronize()

    # ---- timed region: exactly K whole steps, synchronised on both sides
    t0 = time.perf_counter()
    run("timed", timed_idx)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    got_out = (out_c if args.path == "chunk" else out).cpu().numpy()

    # ---- decode-call duration by HIP events (split-K kernel + LSE merge each, a new cache
    # copy each, back to back)
    flush_infinity_cache()
    n_calls = calls_to_time(n_copies)
    dec_ms, dec_how = call_time(decode_call, caches, n_calls)
    one_call_us = single_call_us(decode_call, caches)
    ms_per_step = (t1 - t0) * 1e3 / K
    token_heads = int(L.sum()) * w.num_kv_heads
    value = token_heads / (ms_per_step * 1e-3)

    alg = algorithmic_bytes(w, L)
    achieved = alg / (dec_ms * 1e-3) / 1e9
    ceiling = stream_read_ceiling()
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "read_ceiling": ceiling, "frac_of_read_ceiling": achieved / ceiling["achieved"],
            # counters are recorded for the default route (tq_decode_step, MFMA kernel) only
            "traffic": recorded_traffic(w.name) if args.path == "step" and not args.formats else None,
            "kernel": {"step": "tq_decode_step", "fused": "tq_decode_attention_fused",
                       "separate": "tq_decode_attention", "chunk": "tq_decode_chunk_fused"}[args.path]
            + (" (decode_ref_kernel" if args.variant == 1 else " (decode_mfma_kernel")
            + " + combine_kernel)",
            "call_us": dec_ms * 1e3,
            **dec_how,
            "single_call_us": one_call_us,
            "algorithmic_bytes_per_call": alg}
    exact = args.path != "chunk" and args.q_scale == 1.0 and not args.v_skip_threshold \
        and not args.k_skip_threshold
    cpu, parity = None, None
    codebooks = None
    if not args.no_cpu_baseline:
        from tests.conftest import load_codebook
        codebooks = {"turbo3": load_codebook("turbo3"), "turbo4": load_codebook("turbo4")}
        cpu, o_ref = cpu_baseline(w, args.workload, formats, seed, args.cpu_seconds)
        # Exactness gate: the timed steps' output for sequence 0 (every cache copy holds the
        # same tokens, so the last step's output is the step's) against the oracle's output of
        # the same step, at the parity bars of the tests.  Only where the step is the oracle's:
        # exact attention, unscaled queries, one query position.
        if exact:
            parity = oracle_parity(master, w, 0, int(L[0]), k_list[0], v_list[0], q_np[0], got_out[0], o_ref=o_ref,
                                   codebooks=codebooks)
    per_workload = None
    if not args.no_extra and args.workload == 1 and args.path == "step" and exact and not args.formats:
        del caches, k_list, v_list
        torch.cuda.empty_cache()
        per_workload = {w.name: {"call_us": dec_ms * 1e3, "single_call_us": one_call_us,
                                 "algorithmic_bytes_per_call": alg,
                                 "achieved_GBs": achieved, "frac": achieved / HBM_PEAK_GBS,
                                 "frac_of_read_ceiling": achieved / ceiling["achieved"],
                                 "kv_token_heads_per_s": token_heads / (dec_ms * 1e-3),
                                 "q_token_heads_per_s": token_heads * w.group / (dec_ms * 1e-3),
                                 "traffic": roof["traffic"], "parity": parity, "cpu_baseline": cpu}}
        for widx in EXTRA_WORKLOADS:
            name, rec = extra_workload(widx, seed, not args.no_cpu_baseline, codebooks, ceiling["achieved"],
                                       args.extra_cpu_seconds)
            per_workload[name] = rec
            print(f"bench.py: {name} {rec['call_us']:.1f} us per call, {rec['frac']:.3f} of 8 TB/s",
                  file=sys.stderr, flush=True)
    line = {
        "metric": METRIC, "value": value, "unit": "KV token-heads/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": ms_per_step,
        "value_per_query_head": value * w.group,     # the same rate counted per query head (x G)
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8 codes, f32 valu" if args.variant == 1 else "u8 codes, f16 mfma, f32 accumulate",
        "data": "synthetic (seeded; no model weights)",
        "config": {"workload": w.name, "batch": w.batch, "num_q_heads": Hq, "num_kv_heads": w.num_kv_heads,
                   "context_total": int(L.sum()), "k_format": w.k_format, "v_format": w.v_format,
                   "cache_copies": n_copies, "graph": use_graph,
                   "path": args.path, "variant": args.variant,
                   "v_skip_threshold": args.v_skip_threshold, "k_skip_threshold": args.k_skip_threshold,
                   "q_scale": args.q_scale,
                   "q_len": args.q_len if args.path == "chunk" else 1},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
        "per_workload": per_workload,
    }
    print(json.dumps(line), flush=True)
    bad = [p for p in [parity] + [r["parity"] for r in (per_workload or {}).values()] if p is not None and not p["ok"]]
    if bad:
        print(f"bench.py: outside the parity bars: {bad}", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
