"""Paged decode attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2|4|5|6|7]
                    [--kernel auto|mfma|valu] [--partition P] [--bucket B]

A step is one pass of the hot path over one batch:
  config 5 (default; the full Llama-3-8B-shaped decode step, attention only:
      32 layers, each with its own KV pool, bucket B = 256 rows of which the
      seeded real rows have L ~ U[1, 8192] and the rest are padded at L = 0,
      one [B, 512] table for every layer): pa_decode for each of the 32
      layers, with the balanced split (partition_tokens 0, the library's
      default; --partition 512 runs the fixed 512-token split instead);
  config 2 (Llama-3-8B-shaped layer, B = 64, L ~ U[128, 4096]):
      the KV append of the 64 new tokens and pa_decode over all 64 rows,
      as pa_write_kv then pa_decode (--step separate, the default) or as
      one pa_decode_append call (--step fused); the line reports the other
      form's step time too;
  config 4 (Llama-3.3-70B-shaped layer, B = 256, lognormal lengths):
      pa_decode;
  config 6 (chunked prefill on an 8B-shaped layer: 8 prompts, one 512-token
      chunk each, 0 .. 3,584 tokens already cached):
      pa_write_kv of the 4,096 chunk tokens, then pa_prefill; its roofline is
      the matrix cores' (bf16 dense), in TFLOP/s;
  config 7 (MLA-style latent decode on a DeepSeek-V3-shaped layer: 128 heads
      over one 576-element latent per token, 64-token pages, B = 256 with
      the 70B batch's lengths): pa_latent_decode; HBM roofline, with the
      matrix cores' share reported beside it.
Copy-on-write block copies fire only on a divergent write to a shared block,
which these batches do not have; pa_copy_blocks is timed separately
(`copy_blocks_us`) on one 8B-shaped block pair per call.

Inputs are seeded, synthetic and resident in HBM before timing; three
independent copies of the inputs rotate so that no step reads data the
previous one left in the 256 MB last-level cache (config 5 streams > 0.5 GB
per step by itself and uses one copy).

Printed: one JSON line with the achieved KV bandwidth (valid tokens' K and V
bytes / step time), sequences per second per layer, the roofline of the
attention call (algorithmic bytes, or flops, per call / its mean duration:
HIP events on the launch stream around back-to-back calls, which for the
decode-only steps is the timed region itself), and the CPU oracle timed on a
bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_TFLOPS = 2500.0  # dense bf16 matrix-core peak
METRIC = "paged decode attention: achieved KV GB/s (% of HBM peak) and seqs/s per layer"
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SRC = {
    "mfma": ["decode_mfma.hip", "device_common.h", "worklist.h", "launch.h"],
    "valu": ["decode_valu.hip", "decode_reduce.hip", "device_common.h", "worklist.h", "launch.h"],
    "latent": ["latent_mfma.hip", "lds_stream.h", "mfma_tile.h", "device_common.h", "worklist.h",
               "launch.h"],
    "prefill": ["prefill_mfma.hip", "lds_stream.h", "mfma_tile.h", "device_common.h", "worklist.h",
                "launch.h"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=5, choices=[2, 4, 5, 6, 7])
    ap.add_argument("--kernel", default="auto", choices=["auto", "mfma", "valu"])
    ap.add_argument("--partition", type=int, default=-1,
                    help="split-K partition tokens; 0 = balanced split; -1 = the library's "
                         "choice from the dims (the default: fixed partitions of 256 tokens "
                         "for one row, 192 for two, 320 for three or four, 384 for five to "
                         "eight; the balanced split above)")
    ap.add_argument("--bucket", type=int, default=256, help="config 5 batch bucket")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--block-size", type=int, default=16,
                    help="tokens per KV block for the 8B/70B layers (8 .. 256; other than 16 "
                         "needs the balanced split)")
    ap.add_argument("--placement", default="random", choices=["random", "contiguous"],
                    help="physical block placement of the 8B/70B layers")
    ap.add_argument("--kv-layout", default="paged", choices=["paged", "contiguous"],
                    help="8B/70B layers: the paged pool, or the same values in an unpaged "
                         "cache decoded by pa_decode_contiguous (no table; the step is the "
                         "decode alone)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed steps in a HIP graph (one step per input copy) "
                         "and time its replays")
    ap.add_argument("--step", default="separate", choices=["fused", "separate"],
                    help="8B batch: append + decode in one call, or two calls")
    ap.add_argument("--no-other-form", action="store_true",
                    help="8B batch: do not also time the other form of the step (profiling)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU work budget for the oracle baseline (0 = skip)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="also run a plain copy kernel of known size (counter calibration)")
    ap.add_argument("--spike-rows", type=int, default=0,
                    help="config 7: rows (of those longer than two tiles) whose last latent "
                         "is made to outscore their first tiles by far, so that they take "
                         "the exact recompute (-1 = all of them)")
    return ap.parse_args()


def kernel_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRC[kernel]:
        with open(os.path.join(ROOT, "paged_kv_cache_55_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per decode call from a committed counter summary, if the
    kernel sources still hash to what was profiled."""
    path = os.path.join(PROFILE_DIR, f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("TRAFFIC_JSON "):
            rec = json.loads(line[len("TRAFFIC_JSON "):])
            if rec.get("kernel_hash") == kernel_hash(kernel):
                return rec.get("hbm_bytes_per_call")
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not "
              "supported (the paged decode path shards by sequence or KV head "
              "with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import paged_kv_cache_55_amd as pk
    import workloads as wl

    if not os.path.exists(os.path.join(ROOT, "paged_kv_cache_55_amd", "libpagedkv.so")):
        from paged_kv_cache_55_amd import build as b
        b.build()
    pk.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kernel = args.kernel if args.kernel != "auto" else "mfma"
    part = part_call = args.partition  # part: as reported; part_call: what the calls pass
    split_policy = "library choice (PA_PARTITION_AUTO)" if part == pk.PARTITION_AUTO else "explicit"

    # ---------------- inputs ----------------
    if args.config in (2, 4):
        mk = wl.config2 if args.config == 2 else wl.config4
        case = mk(block_size=args.block_size, placement=args.placement)
        copies = [case.to(dev) for _ in range(max(1, args.copies))]
        B, Hq, Hkv, D = case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim
        n_real = int((case.seq_lens > 0).sum())
        kv_bytes = case.kv_bytes()
        layers = 1
        lens_host = case.seq_lens.numpy()
        workload = ("llama3_8b_layer_b64_u128_4096" if args.config == 2
                    else "llama33_70b_layer_b256_lognormal1024")
        if args.block_size != 16:
            workload += f"_block{args.block_size}"
        if args.placement != "random":
            workload += f"_{args.placement}"
        contiguous_kv = args.kv_layout == "contiguous"
        if contiguous_kv:
            workload += "_contiguous_kv"
            unpaged = [wl.contiguous_cache(c) for c in copies]
        outs = [torch.empty_like(c.q) for c in copies]
        dims = pk.make_dims(B, Hq, Hkv, D, case.max_blocks_per_seq, case.num_blocks,
                            pk.PA_BF16, part, kernel, case.block_size)
        ws_bytes = pk.pa_decode_workspace_bytes(dims)
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        scale = case.scale

        def decode_calls(i):
            c = copies[i % len(copies)]
            if contiguous_kv:
                kc, vc = unpaged[i % len(copies)]
                return [(c.q, kc, vc, None, c.seq_lens, outs[i % len(copies)])]
            return [(c.q, c.k_pool, c.v_pool, c.block_tables, c.seq_lens, outs[i % len(copies)])]

        def pre(i):
            c = copies[i % len(copies)]
            if c.slot_mapping is not None and not contiguous_kv:
                pk.pa_write_kv(c.k_new, c.v_new, c.slot_mapping, c.k_pool, c.v_pool)
    elif args.config == 6:
        case = wl.prefill_step_8b(block_size=args.block_size)
        copies = [case.to(dev) for _ in range(max(1, args.copies))]
        Hq, Hkv, D = case.num_q_heads, case.num_kv_heads, case.head_dim
        B = n_real = int(case.seq_lens.shape[0])  # sequences (q holds their chunk rows)
        kv_bytes = case.kv_bytes()
        layers = 1
        lens_host = case.seq_lens.numpy()
        workload = "prefill_step_llama3_8b_8x512"
        if args.block_size != 16:
            workload += f"_block{args.block_size}"
        outs = [torch.empty_like(c.q) for c in copies]
        ws = None
        scale = case.scale

        def decode_calls(i):
            c = copies[i % len(copies)]
            return [(c.q, c.k_pool, c.v_pool, c.block_tables, c.seq_lens, outs[i % len(copies)])]

        def pre(i):
            c = copies[i % len(copies)]
            pk.pa_write_kv(c.k_new, c.v_new, c.slot_mapping, c.k_pool, c.v_pool)
    elif args.config == 7:
        case = wl.latent_decode_batch()
        spiked = []
        if args.spike_rows:
            spiked = spike_latent_rows(case, args.spike_rows)
        copies = [case.to(dev) for _ in range(max(1, args.copies))]
        B, Hq, Hkv, D = case.q.shape[0], case.q.shape[1], 1, case.q.shape[2]
        n_real = int((case.seq_lens > 0).sum())
        kv_bytes = case.kv_bytes()
        layers = 1
        lens_host = case.seq_lens.numpy()
        workload = "deepseek_v3_mla_layer_b256_lognormal1024"
        if spiked:
            workload += f"_spiked{len(spiked)}"
        outs = [torch.empty((B, Hq, wl.LATENT_VALUE_DIM), dtype=torch.bfloat16, device=dev)
                for _ in copies]
        ldims = pk.make_latent_dims(B, case.block_tables.shape[1], case.kv_pool.shape[0])
        ws = torch.zeros(pk.pa_latent_workspace_bytes(ldims), dtype=torch.uint8, device=dev)
        scale = case.scale
        kernel = "latent"

        def decode_calls(i):
            c = copies[i % len(copies)]
            return [(c.q, c.kv_pool, None, c.block_tables, c.seq_lens, outs[i % len(copies)])]

        def pre(i):
            pass
    else:
        spec = wl.config5_spec(args.bucket)
        B, Hq, Hkv, D = spec.bucket, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
        n_real = spec.n_real
        layers = spec.layers
        kv_bytes = spec.kv_bytes_per_layer() * layers
        lens_host = spec.seq_lens
        workload = f"llama3_8b_step_32layers_bucket{args.bucket}"
        bt = torch.from_numpy(spec.block_tables).to(dev)
        lens = torch.from_numpy(spec.seq_lens).to(dev)
        layer_t = [wl.config5_layer(spec, l, dev) for l in range(layers)]
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
        dims = pk.make_dims(B, Hq, Hkv, D, wl.C5_MB, spec.num_blocks, pk.PA_BF16, part, kernel)
        ws_bytes = pk.pa_decode_workspace_bytes(dims)
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        scale = 1.0 / math.sqrt(D)
        case = None
        copies = []

        def decode_calls(i):
            return [(q, k, v, bt, lens, out) for (q, k, v) in layer_t]

        def pre(i):
            pass

    if part == pk.PARTITION_AUTO:  # the library's rule, which only the dims decide
        fixed = kernel != "mfma" or (
            B <= 8 and (case is None or case.block_size == 16)
            and not (args.config in (2, 4) and args.kv_layout == "contiguous"))
        mfma_part = 256 if B <= 1 else 192 if B == 2 else 320 if B <= 4 else 384
        part = (mfma_part if kernel == "mfma" else 512) if fixed and args.config not in (6, 7) \
            else 0
    if part > 0:
        workload += f"_split{part}"
    stream = torch.cuda.current_stream()

    def step(i, events=None, mode=None):
        mode = mode or args.step
        fused = mode == "fused" and args.config == 2 and args.kv_layout == "paged"
        stream = torch.cuda.current_stream()  # the capture stream inside a graph capture
        if not fused:
            pre(i)
        for (q, k, v, tb, ln, o) in decode_calls(i):
            if events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            if fused:
                c = copies[i % len(copies)]
                pk.pa_decode_append(q, c.k_new, c.v_new, c.slot_mapping, k, v, tb, ln, scale, o,
                                    partition_tokens=part_call, kernel=kernel, workspace=ws,
                                    stream=stream)
            elif args.config == 6:
                pk.pa_prefill(q, k, v, tb, ln, copies[i % len(copies)].query_start, scale, o,
                              stream=stream)
            elif args.config == 7:
                pk.pa_latent_decode(q, k, tb, ln, scale, o, workspace=ws, stream=stream)
            elif tb is None:
                pk.pa_decode_contiguous(q, k, v, ln, scale, o, workspace=ws, stream=stream)
            else:
                pk.pa_decode(q, k, v, tb, ln, scale, o, partition_tokens=part_call, kernel=kernel,
                             workspace=ws, stream=stream)
            if events is not None:
                e1.record(stream)
                events.append((e0, e1))

    def timed_steps(mode):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        if args.graph:
            # one graph holds one step per input copy; replays cover the steps
            per_graph = len(copies) if copies else 1
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(per_graph):
                    step(i, mode=mode)
            replays = max(1, args.steps // per_graph)
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            t0.record(stream)
            for _ in range(replays):
                g.replay()
            t1.record(stream)
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) / (replays * per_graph)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(args.steps):
            step(i, mode=mode)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    # ---------------- timing ----------------
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = timed_steps(args.step)
    other_ms = None
    if args.config == 2 and not args.no_other_form and args.kv_layout == "paged":
        # the other form, for comparison
        other = "separate" if args.step == "fused" else "fused"
        for i in range(args.warmup):
            step(i, mode=other)
        other_ms = timed_steps(other)

    # The attention call's mean duration for the roofline: HIP events on the
    # launch stream around back-to-back calls. A decode-only step (configs 4,
    # 5 and 7, eager) is exactly that, so its timed region is used as is;
    # steps that also append K/V (configs 2 and 6) or run as a graph get a
    # pass of their own with the calls alone.
    calls_per_step = len(decode_calls(0))
    decode_only = args.config in (4, 5, 7) and not args.graph
    if decode_only:
        kernel_ms = ms_per_step / calls_per_step
    else:
        saved_pre = pre
        pre = lambda i: None  # noqa: E731  the calls alone (a fused call keeps its append)
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        ka = torch.cuda.Event(enable_timing=True)
        kb = torch.cuda.Event(enable_timing=True)
        ka.record(stream)
        for i in range(args.steps):
            step(i)
        kb.record(stream)
        torch.cuda.synchronize()
        kernel_ms = ka.elapsed_time(kb) / (args.steps * calls_per_step)
        pre = saved_pre

    # per-call durations with an event pair around each call (a diagnostic:
    # the events add their own gaps)
    events = []
    for i in range(args.steps):
        step(i, events)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in events])

    # copy-on-write block copy, one 8B-shaped block pair per call
    copy_us = None
    if args.config in (2, 4):
        c = copies[0]
        pair = torch.tensor([[int(c.block_tables[0, 0]), c.poison_block]], dtype=torch.int32,
                            device=dev)
        ce0 = torch.cuda.Event(enable_timing=True)
        ce1 = torch.cuda.Event(enable_timing=True)
        kp = c.k_pool.clone()
        vp = c.v_pool.clone()
        for _ in range(5):
            pk.pa_copy_blocks(kp, vp, pair)
        ce0.record(stream)
        for _ in range(50):
            pk.pa_copy_blocks(kp, vp, pair)
        ce1.record(stream)
        torch.cuda.synchronize()
        copy_us = ce0.elapsed_time(ce1) / 50 * 1e3
        del kp, vp

    if args.traffic_probe:
        n = 1 << 28
        x = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(f"TRAFFIC_PROBE neg bytes_read={n} bytes_written={n}", file=sys.stderr)

    # ---------------- figures ----------------
    sec = ms_per_step / 1e3
    value = kv_bytes / sec / 1e9
    bsz = (case.block_size if args.config != 7 else wl.LATENT_BLOCK) if case is not None else 16
    table_bytes = int(sum(math.ceil(int(L) / bsz) for L in lens_host)) * 4
    unpaged_kv = args.config in (2, 4) and args.kv_layout == "contiguous"
    if unpaged_kv:
        table_bytes = 0  # no table is read
    per_call_alg = (kv_bytes / layers) + 2 * B * Hq * D * 2 + table_bytes + 4 * B
    latent_flops = None
    if args.config == 7:  # q read, out written (512 of 576 elements), latents, tables
        per_call_alg = kv_bytes + B * Hq * (D + wl.LATENT_VALUE_DIM) * 2 + table_bytes + 4 * B
        # scores: 2 * 576 flops, values: 2 * 512 flops per (head, cached token)
        latent_flops = int(lens_host.sum()) * Hq * 2 * (D + wl.LATENT_VALUE_DIM)
    fused = args.config == 2 and args.step == "fused" and not unpaged_kv
    if fused:  # the appended tokens: k_new/v_new read, their slots written, slot ids
        T = int((case.slot_mapping >= 0).sum())
        per_call_alg += 4 * T * Hkv * D * 2 + 4 * B
    mean_call_s = kernel_ms / 1e3
    achieved = per_call_alg / mean_call_s / 1e9
    traffic = load_traffic(kernel, workload)
    prefill_flops = None
    if args.config == 6:  # QK and PV: 2 D flops each per (query head, key) pair
        qs = case.query_start.numpy()
        # bytes: every row's K/V once, the chunk rows' queries read and
        # outputs written, tables, lengths and row starts
        per_call_alg = (kv_bytes / layers + 2 * int(qs[-1]) * Hq * D * 2 + table_bytes
                        + 4 * B + 4 * (B + 1))
        prefill_flops = 0
        for s_i, L in enumerate(lens_host.tolist()):
            n = int(qs[s_i + 1] - qs[s_i])
            keys = n * (L - n) + n * (n + 1) // 2  # sum over chunk rows of (p + 1)
            prefill_flops += 4 * Hq * D * keys
        achieved = prefill_flops / mean_call_s / 1e12
        traffic = load_traffic("prefill", workload)
    mfma_share = None
    if latent_flops is not None:
        mfma_share = {"achieved_tflops": round(latent_flops / mean_call_s / 1e12, 1),
                      "peak_tflops": MFMA_BF16_TFLOPS,
                      "frac": round(latent_flops / mean_call_s / 1e12 / MFMA_BF16_TFLOPS, 4),
                      "flops_per_call": latent_flops}

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if args.cpu_seconds > 0:
        if args.config == 5:
            cpu = cpu_baseline_step(args, spec, layer_t, workload)
        else:
            cpu = cpu_baseline(args, case, lens_host, kv_bytes / layers, workload)
        cpu.update(host_threads())

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) values, seeded lengths and block placement)",
        "config": {
            "workload": workload,
            "batch": B, "real_rows": n_real, "q_heads": Hq, "kv_heads": Hkv,
            "head_dim": D, "layers": layers,
            "block_size": bsz,
            "placement": args.placement if case is not None else "random",
            "partition_tokens": part, "split_policy": split_policy, "kernel": kernel,
            "graph": args.graph,
            "kv_bytes_per_step": kv_bytes,
            "step": ("pa_decode_contiguous (unpaged cache, no table; no append)" if unpaged_kv
                     else "pa_decode_append (64-token KV append fused into the decode)"
                     if fused else "pa_write_kv(64 tokens) + pa_decode" if args.config == 2
                     else "pa_decode" if args.config == 4
                     else "pa_write_kv(4096 chunk tokens) + pa_prefill" if args.config == 6
                     else "pa_latent_decode" if args.config == 7
                     else "32 x pa_decode"),
        },
        "other_step_form_ms": None if other_ms is None else {
            ("separate" if args.step == "fused" else "fused"): round(other_ms, 5)},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seqs_per_s_per_layer": round(n_real * layers / sec, 1) if layers == 1 else round(n_real / (sec / layers), 1),
        "decode_call_us": {"mean": round(float(call_ms.mean()) * 1e3, 2),
                           "p10": round(float(np.percentile(call_ms, 10)) * 1e3, 2),
                           "p50": round(float(np.percentile(call_ms, 50)) * 1e3, 2),
                           "p90": round(float(np.percentile(call_ms, 90)) * 1e3, 2)},
        "copy_blocks_us": None if copy_us is None else round(copy_us, 2),
        "roofline": {
            "kernel": (f"prefill_mfma_kernel<{D}>" if args.config == 6 else
                       "latent_decode_kernel + latent_merge_kernel (one call: the decode, then "
                       "the merge of cut rows)"
                       if args.config == 7 else
                       f"decode_mfma_balanced_kernel<{D}, contiguous> (unpaged cache; no table)"
                       if unpaged_kv else
                       roofline_kernel(kernel, part, D) + (" with the fused KV append"
                                                           if fused else "")),
            "bound": "mfma" if args.config == 6 else "hbm",
            "achieved": round(achieved, 1),
            "peak": MFMA_BF16_TFLOPS if args.config == 6 else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if args.config == 6 else "GB/s",
            "frac": round(achieved / (MFMA_BF16_TFLOPS if args.config == 6 else HBM_PEAK_GBS), 4),
            "traffic": traffic,
            "algorithmic_bytes_per_call": int(per_call_alg),
            "algorithmic_flops_per_call": prefill_flops,
            "matrix_cores": mfma_share,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def roofline_kernel(kernel: str, part: int, head_dim: int) -> str:
    """Which launches one pa_decode call makes."""
    if kernel == "mfma" and part == 0:
        return (f"decode_mfma_balanced_kernel<{head_dim}> (one launch per call; "
                "cut pairs are merged inside it)")
    if kernel == "mfma":
        return (f"decode_mfma_kernel<{head_dim}> (one launch per call; a row's partitions "
                "are merged inside it by the last one to finish)")
    return f"decode_valu_kernel<{head_dim}> + decode_reduce_kernel when a row spans several partitions"


def host_threads():
    """What the host offers and what the oracle used: every timed oracle call
    runs under a BLAS limit of one thread (numpy's matrix products), and the
    oracle itself is single-threaded Python."""
    from threadpoolctl import threadpool_info
    return {"host_cpus": os.cpu_count(),
            "blas_threads": 1,
            "blas_libraries": sorted({i.get("internal_api", "?") for i in threadpool_info()})}


def spike_latent_rows(case, n):
    """Makes the last latent of `n` rows (evenly spaced among the rows longer
    than two 32-token tiles; all of them for n < 0) equal 5 x the query of
    head 0: that head's score there exceeds the rest of the row by about 120
    natural-log units, so the piece holding it flags the row (unless the
    token opens that piece) and the row takes the exact recompute. Returns
    the rows."""
    import numpy as np
    lens = case.seq_lens.numpy()
    cand = [b for b in range(len(lens)) if lens[b] > 64]
    if n >= 0 and n < len(cand):
        cand = [cand[i] for i in np.linspace(0, len(cand) - 1, n).round().astype(int)]
    bs = case.kv_pool.shape[1]
    for b in cand:
        t = int(lens[b]) - 1
        blk = int(case.block_tables[b, t // bs])
        case.kv_pool[blk, t % bs] = (5.0 * case.q[b, 0].float()).to(case.kv_pool.dtype)
    return cand


def cpu_baseline_step(args, spec, layer_t, workload):
    """The float64 oracle on one host core over a sample of the 32-layer step:
    16 real rows (seeded) of 4 layers (0, 10, 21, 31), the sample repeated
    until the time budget is spent. Each (layer, row set) gets a host copy of
    just the blocks its rows reference, made before timing; the oracle's own
    table walk over that copy is timed. The rate (KV bytes per second) gives
    the time of the whole step."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads import to_numpy

    rng = np.random.default_rng(55_005)
    rows = sorted(rng.choice(spec.n_real, size=min(16, spec.n_real), replace=False).tolist())
    layers = [l for l in (0, 10, 21, 31) if l < len(layer_t)]
    elem, Hkv, D = 2, spec.num_kv_heads, spec.head_dim
    samples = []
    for l in layers:
        q, k, v = layer_t[l]
        need = sorted({int(spec.block_tables[b, j]) for b in rows
                       for j in range(math.ceil(int(spec.seq_lens[b]) / 16))})
        remap = np.zeros(spec.num_blocks, dtype=np.int64)
        remap[need] = np.arange(len(need))
        idx = torch.tensor(need, dtype=torch.long, device=k.device)
        samples.append(dict(q=to_numpy(q[rows]), k_pool=to_numpy(k[idx]), v_pool=to_numpy(v[idx]),
                            block_tables=remap[spec.block_tables[rows]].astype(np.int32),
                            seq_lens=spec.seq_lens[rows], scale=1.0 / math.sqrt(D),
                            dtype="bf16"))
    sample_bytes = int(spec.seq_lens[rows].astype(np.int64).sum()) * Hkv * D * 2 * elem
    done_bytes, done_decodes, t_total, passes = 0, 0, 0.0, 0
    with threadpool_limits(limits=1):
        while t_total < args.cpu_seconds:
            for a in samples:
                t = time.perf_counter()
                oracle.paged_decode(**a)
                t_total += time.perf_counter() - t
                done_bytes += sample_bytes
                done_decodes += len(rows)
            passes += 1
    rate = done_bytes / t_total
    return {
        "value": round(rate / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{len(rows)} real rows x {len(layers)} layers ({layers}) of {workload}, "
                  f"{passes} pass(es): {done_decodes} sequence decodes, "
                  f"{done_bytes / 1e6:.1f} MB of K/V in {t_total:.1f} s, float64 numpy, "
                  "BLAS limited to 1 thread; the step time is scaled by K/V bytes",
        "seqs_per_s": round(done_decodes / t_total, 2),
        "step_s": round(spec.kv_bytes_per_layer() * len(layer_t) / rate, 2),
    }


def cpu_baseline(args, case, lens_host, kv_bytes_per_layer, workload):
    """Time the float64 oracle on host cores over a bounded sample."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads as wl
    from workloads import to_numpy

    if isinstance(case, wl.LatentCase):
        return cpu_baseline_latent(args, case, lens_host, workload)
    if case.query_start is not None:
        return cpu_baseline_prefill(args, case, kv_bytes_per_layer, workload)
    a = dict(q=to_numpy(case.q), k_pool=to_numpy(case.k_pool), v_pool=to_numpy(case.v_pool),
             block_tables=to_numpy(case.block_tables), seq_lens=to_numpy(case.seq_lens),
             scale=case.scale, dtype=case.dtype)
    rows_all = list(range(case.num_seqs))
    done_bytes, done_rows, t_total = 0, 0, 0.0
    elem = 2
    with threadpool_limits(limits=1):
        i = 0
        while t_total < args.cpu_seconds:
            b = rows_all[i % len(rows_all)]
            t = time.perf_counter()
            oracle.paged_decode(**a, rows=[b])
            t_total += time.perf_counter() - t
            done_bytes += int(lens_host[b]) * case.num_kv_heads * case.head_dim * 2 * elem
            done_rows += 1
            i += 1
    return {
        "value": round(done_bytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done_rows} sequence decodes of {workload} (rows in batch order, "
                  f"{done_bytes / 1e6:.1f} MB of K/V) in {t_total:.1f} s, float64 numpy, "
                  "BLAS limited to 1 thread",
        "seqs_per_s": round(done_rows / t_total, 2),
    }


def cpu_baseline_latent(args, case, lens_host, workload):
    """The float64 latent-decode oracle on one host core, one row at a time
    (rows in batch order) until the time budget is spent."""
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads import to_numpy

    q, kv = to_numpy(case.q), to_numpy(case.kv_pool)
    bt, lens = to_numpy(case.block_tables), to_numpy(case.seq_lens)
    done_bytes, done_rows, t_total = 0, 0, 0.0
    with threadpool_limits(limits=1):
        while t_total < args.cpu_seconds:
            b = done_rows % len(lens_host)
            t = time.perf_counter()
            oracle.latent_decode(q, kv, bt, lens, case.scale, case.dtype, rows=[b])
            t_total += time.perf_counter() - t
            done_bytes += int(lens_host[b]) * kv.shape[2] * 2
            done_rows += 1
    return {
        "value": round(done_bytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done_rows} row decodes of {workload} (rows in batch order, "
                  f"{done_bytes / 1e6:.1f} MB of latents) in {t_total:.1f} s, float64 numpy, "
                  "BLAS limited to 1 thread",
        "seqs_per_s": round(done_rows / t_total, 2),
    }


def cpu_baseline_prefill(args, case, kv_bytes, workload):
    """The float64 chunked-prefill oracle on one host core, one whole
    sequence at a time until the time budget is spent; its (query, key)
    rate gives the time of the whole step."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads import to_numpy

    k, v = oracle.write_kv(to_numpy(case.k_pool), to_numpy(case.v_pool), to_numpy(case.k_new),
                           to_numpy(case.v_new), to_numpy(case.slot_mapping),
                           block_size=case.block_size)
    q, bt, lens = to_numpy(case.q), to_numpy(case.block_tables), to_numpy(case.seq_lens)
    qs = to_numpy(case.query_start)
    keys = []
    for s_i, L in enumerate(lens.tolist()):
        n = int(qs[s_i + 1] - qs[s_i])
        keys.append(n * (L - n) + n * (n + 1) // 2)
    done_keys, t_total, seqs = 0, 0.0, 0
    with threadpool_limits(limits=1):
        while t_total < args.cpu_seconds:
            s_i = seqs % len(lens)
            t = time.perf_counter()
            oracle.paged_prefill(q, k, v, bt, lens, qs, case.scale, case.dtype,
                                 block_size=case.block_size, seqs=[s_i])
            t_total += time.perf_counter() - t
            done_keys += keys[s_i]
            seqs += 1
    step_s = t_total * sum(keys) / done_keys
    return {
        "value": round(kv_bytes / step_s / 1e9, 6),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{seqs} whole-sequence chunks of {workload} ({done_keys} query-key pairs "
                  f"of {sum(keys)} per step) in {t_total:.1f} s, float64 numpy, BLAS limited "
                  "to 1 thread; the step time is scaled by query-key pairs",
        "step_s": round(step_s, 3),
    }


if __name__ == "__main__":
    main()
