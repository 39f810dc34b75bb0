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
of the model).  Steps are captured in a HIP graph and replayed, so host launch
overhead is not in the timed region.

Prints ONE JSON line.  value = KV token-heads per second of whole steps
(visible tokens x KV heads / step time).  roofline = the decode call
(split-K kernel + LSE combine) timed by HIP events on its stream around a run of
calls enqueued eagerly behind a GPU sleep, so they run back to back: algorithmic
packed K+V bytes per call / average call duration (both kernels of the call),
against 8 TB/s.
cpu_baseline = the float64 oracle (oracle/) doing the same step on a bounded
sample, on the host cores; its output for sequence 0 also gates the run: the
GPU's output of the timed step must sit within the tests' parity bars (rel-L2
1e-3, max-abs 5e-3), reported as "parity", or bench.py exits non-zero.
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


def parse():
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
    return p.parse_args()


KERNEL_SOURCES = tuple("quantized_kv_cache_decode_amd/csrc/" + f
                       for f in ("decode_mfma.hip", "decode_ref.hip", "combine.hip", "tq_device.h", "tq_encode.h",
                                 "tq_launch.h"))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash():
    """sha256 of the decode and merge kernel sources (ties recorded counters to the code)."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload_name):
    """HBM bytes per decode call from the committed FETCH_SIZE/WRITE_SIZE profile, or None
    when there is none for this workload or the kernels changed since it was taken."""
    import json
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


def cpu_baseline(w, seed, budget_s):
    """The oracle doing the same step (append one token, full-dequant attention) on host cores.

    Returns (record, o): the baseline record and the oracle's float64 output [Hq, 128] of
    sequence 0, against which main() checks the GPU's output of the same step."""
    from threadpoolctl import threadpool_info

    from oracle import codec, reference
    from synth import kv_slice, new_token_kv, queries, sign_vector
    from synth.gen import context_lengths
    from tests.conftest import load_codebook
    cbs = {"turbo3": load_codebook("turbo3"), "turbo4": load_codebook("turbo4")}
    sk, sv = sign_vector(seed, "k"), sign_vector(seed, "v")
    b = 0
    L = int(context_lengths(w, seed)[b])   # sequence 0's visible tokens after the step's append
    pre = L - 1
    k16 = np.stack([kv_slice(w, seed, "k", b, h, pre) for h in range(w.num_kv_heads)])
    v16 = np.stack([kv_slice(w, seed, "v", b, h, pre) for h in range(w.num_kv_heads)])
    enc = reference.encode_sequence(k16, v16, w.k_format, w.v_format, sk, sv, cbs, capacity=((L + 31) // 32) * 32)
    kn = np.stack([new_token_kv(w, seed, "k", b, h, 0) for h in range(w.num_kv_heads)])
    vn = np.stack([new_token_kv(w, seed, "v", b, h, 0) for h in range(w.num_kv_heads)])
    q = queries(w, seed)[b]
    steps, t0 = 0, time.perf_counter()
    while True:
        # append: encode the new token into slot L-1
        if w.k_format == "f16":
            enc["k_f16"][:, pre] = kn[:, 0]
        else:
            c, n = codec.encode(kn, sk, cbs[w.k_format])
            enc["k_codes"][:, pre], enc["k_norms"][:, pre] = c[:, 0], n[:, 0]
        c, n = codec.encode(vn, sv, cbs[w.v_format])
        enc["v_codes"][:, pre], enc["v_norms"][:, pre] = c[:, 0], n[:, 0]
        k_hat, v_hat = reference.dequant_sequence(enc, w.k_format, w.v_format, sk, sv, cbs, L)
        o = reference.decode_sequence(q, k_hat, v_hat, L)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return o, {
        "value": steps * L * w.num_kv_heads / el,
        "unit": "KV token-heads/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{steps} steps of sequence 0 of {w.name} (append 1 token + float64 full-dequant "
                  f"attention over {L} tokens x {w.num_kv_heads} KV heads x {w.group} query heads each) "
                  f"in {el:.1f} s",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the decode path is built and measured "
              "on a single MI355X; sharding is described, not built.", file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_kv_cache_decode_amd as tq
    from synth import get_workload, new_token_kv, queries
    from tests import support as S
    tq.load_library()
    torch.cuda.set_device(0)
    w = get_workload(args.workload)
    if args.formats:
        from dataclasses import replace
        kf, vf = args.formats.split("/")
        w = replace(w, k_format=kf, v_format=vf)
    seed = 0

    # ---- setup (not timed): prefill L-1 tokens, append the step's token once
    master, k_list, v_list, L, q_np = S.prefill_and_step(w, seed)
    master.v_skip_threshold = args.v_skip_threshold   # (the copies below inherit them)
    master.k_skip_threshold = args.k_skip_threshold
    pre = (L - 1).astype(np.int32)
    per_copy = cache_bytes(master)
    n_copies = max(1, int(math.ceil(args.copies_gib * (1 << 30) / per_copy)))
    caches = [master] + [clone_cache(master) for _ in range(n_copies - 1)]
    kn = S.padded_tensor([np.stack([new_token_kv(w, seed, "k", b, h, 0) for h in range(w.num_kv_heads)])
                          for b in range(w.batch)], 1)
    vn = S.padded_tensor([np.stack([new_token_kv(w, seed, "v", b, h, 0) for h in range(w.num_kv_heads)])
                          for b in range(w.batch)], 1)
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
    del k_list, v_list
    per_graph = n_copies
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

    use_graph = not args.no_graph
    graph = None
    if use_graph:
        try:
            for i in range(per_graph):       # warm the launch path outside capture
                step(i)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(per_graph):
                    step(i)
        except Exception as e:  # pragma: no cover - reported, then eager timing
            print(f"graph capture unavailable ({e!r}); timing eager launches", file=sys.stderr)
            graph, use_graph = None, False

    reps = max(1, args.steps // per_graph) if use_graph else 0
    steps = reps * per_graph if use_graph else args.steps
    warm_reps = max(1, args.warmup // per_graph) if use_graph else 0
    if use_graph:
        for _ in range(warm_reps):
            graph.replay()
    else:
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    # ---- timed region: K whole steps, synchronised on both sides
    t0 = time.perf_counter()
    if use_graph:
        for _ in range(reps):
            graph.replay()
    else:
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # ---- decode-call duration by HIP events on the launch stream.  Events cannot be
    # recorded inside a captured graph here, so the calls are enqueued eagerly behind a
    # GPU sleep long enough for the host to queue them all: they then run back to back
    # (split-K kernel + LSE merge each, a new cache copy each) and one event pair
    # brackets the whole run, so no event sits between two calls' kernels.
    n_calls = min(per_graph, 512)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(5e7))
    ev0.record()
    for i in range(n_calls):
        decode_call(caches[i % n_copies])
    ev1.record()
    torch.cuda.synchronize()
    call_ms = [ev0.elapsed_time(ev1) / n_calls]
    ms_per_step = (t1 - t0) * 1e3 / steps
    token_heads = int(L.sum()) * w.num_kv_heads
    value = token_heads / (ms_per_step * 1e-3)

    alg = algorithmic_bytes(w, L)
    dec_ms = float(np.mean(call_ms)) if call_ms else float("nan")
    achieved = alg / (dec_ms * 1e-3) / 1e9 if call_ms else None
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
            # counters are recorded for the default route (tq_decode_step, MFMA kernel) only
            "traffic": recorded_traffic(w.name) if args.path == "step" and not args.formats else None,
            "kernel": {"step": "tq_decode_step", "fused": "tq_decode_attention_fused",
                       "separate": "tq_decode_attention", "chunk": "tq_decode_chunk_fused"}[args.path]
            + (" (decode_ref_kernel" if args.variant == 1 else " (decode_mfma_kernel")
            + " + combine_kernel)",
            "call_us": dec_ms * 1e3,
            "algorithmic_bytes_per_call": alg}
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        o_ref, cpu = cpu_baseline(w, seed, args.cpu_seconds)
        # Exactness gate: the timed calls' output for sequence 0 (every cache copy holds the
        # same tokens, so the last call's output is the step's) against the oracle's output
        # of the same step, at the parity bars of the tests.  Only where the step is the
        # oracle's: exact attention, unscaled queries, one query position.
        if args.path != "chunk" and args.q_scale == 1.0 and not args.v_skip_threshold and not args.k_skip_threshold:
            rel, mx = S.errors(out[0].cpu().numpy(), o_ref)
            parity = {"sequence": 0, "rel_l2": rel, "max_abs": mx, "rel_l2_bound": 1e-3, "max_abs_bound": 5e-3,
                      "ok": bool(rel <= 1e-3 and mx <= 5e-3)}
    line = {
        "metric": METRIC, "value": value, "unit": "KV token-heads/s", "n_gpus": 1, "steps": steps,
        "warmup": warm_reps * per_graph if use_graph else args.warmup, "ms_per_step": ms_per_step,
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
    }
    print(json.dumps(line), flush=True)
    if parity is not None and not parity["ok"]:
        print(f"bench.py: the timed output of sequence 0 is outside the parity bars: {parity}", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
