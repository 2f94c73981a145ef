"""Decode throughput of the W4 OLMo-3-32B-shaped step on one MI355X.

Workload (default): the full 64-layer random-init stack ([SWA x3, full] x16, d 5,120,
40/8 heads of 128, SwiGLU 27,648, W4 group-128 weights with f16 scales and uint4
zeros), f32 KV cache pre-filled to 16,384 positions in every layer, batch 1, one new
token at position 16,384 (SWA layers read the last 4,096 keys, full layers all
16,385), final RMSNorm, bf16 lm_head 100,278 x 5,120 and greedy argmax. Each step
feeds back the previous step's argmax token. Inputs are seeded synthetic values
resident in HBM before timing starts.

The timed steps replay one step captured in a HIP graph (the position and token live
in device memory); HIP events between the replays give the per-step median, p10 and
p90. Prints one JSON line: tokens/s, ms/step, achieved algorithmic HBM GB/s of the
step, the roofline of the dominant kernel (the gate/up W4 GEMV) measured with
dispatch-stamped HIP events on the launch stream, the read bandwidth a plain
streaming kernel reaches on the same device, the 1,200-token prefill, and the CPU
oracle's throughput on a bounded sample (all host threads and one thread).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode64_16k_hbm_traffic.md")
KERNEL_TRACE_PROFILE = os.path.join(ROOT, "profiles", "decode64_16k_kernel_stats.md")
KERNEL_SOURCES = ["swa_attention_amd/csrc/gemv_core.h", "swa_attention_amd/csrc/decode_kernels.hip",
                  "swa_attention_amd/csrc/decode_kernels.h", "swa_attention_amd/csrc/common.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed PMC summary
    (FETCH_SIZE and WRITE_SIZE, calibrated against a plain copy), or None when the
    kernel sources have changed since the counters were taken."""
    import hashlib
    try:
        line = [l for l in open(TRAFFIC_PROFILE) if l.startswith("traffic-json: ")][0]
    except (OSError, IndexError):
        return None
    rec = json.loads(line[len("traffic-json: "):])
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return rec["bytes_per_launch"] if h.hexdigest()[:16] == rec["source_sha256_16"] else None


def profiled_replay_us():
    """Average gate/up launch duration over the timed graph replays of the committed
    rocprofv3 kernel trace, or None when the kernel sources have changed since."""
    import hashlib
    try:
        line = [l for l in open(KERNEL_TRACE_PROFILE) if l.startswith("roofline-json: ")][0]
    except (OSError, IndexError):
        return None
    rec = json.loads(line[len("roofline-json: "):])
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return rec["graph_replay_avg_us"] if h.hexdigest()[:16] == rec["source_sha256_16"] else None


def host_info():
    """CPU model, logical CPUs and RAM of the host that runs the oracle."""
    model, ram = "unknown", 0.0
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
        ram = next(int(l.split()[1]) for l in open("/proc/meminfo") if l.startswith("MemTotal")) / 2**20
    except (OSError, StopIteration):
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "ram_GiB": round(ram, 1)}


def oracle_block_seconds(config, n_blocks):
    """Seconds of oracle compute for the first n_blocks [SWA,SWA,SWA,full] blocks of a
    workload's decode step (inputs generated outside the timed region)."""
    import oracle as O
    from oracle import runner as R
    from synth import workloads as W
    wl = W.config(config)
    m = wl.model
    x = O.embed(W.embedding_rows(m, wl.seed, R.decode_token(wl), 1)[0])
    t = 0.0
    for l in range(4 * n_blocks):
        T, Kc, Vc = R.layer_inputs(wl, l)
        t0 = time.perf_counter()
        x = O.layer_step(m, m.layer_types[l], T, x, Kc, Vc, wl.n_cached)
        t += time.perf_counter() - t0
        del T, Kc, Vc
    return t


def cpu_baseline(wl, budget_s, config):
    """Oracle (CPU, double accumulation, OpenMP) on whole [SWA,SWA,SWA,full] blocks of
    the same workload until ~budget_s of compute, plus the lm_head; extrapolated to
    the 64-layer token. Input generation is not timed."""
    import numpy as np
    import oracle as O
    from oracle import runner as R
    from synth import workloads as W
    m = wl.model
    x = O.embed(W.embedding_rows(m, wl.seed, R.decode_token(wl), 1)[0])
    t_layers, n_done = 0.0, 0
    while n_done < m.n_layers and t_layers < budget_s:
        for l in range(n_done, n_done + 4):
            T, Kc, Vc = R.layer_inputs(wl, l)
            t0 = time.perf_counter()
            x = O.layer_step(m, m.layer_types[l], T, x, Kc, Vc, wl.n_cached)
            t_layers += time.perf_counter() - t0
            del T, Kc, Vc
        n_done += 4
    lm = W.lm_head_rows(m, wl.seed, 0, m.vocab)
    g = W.final_gain(m, wl.seed)
    t0 = time.perf_counter()
    O.final_logits(x, g, lm, m.eps)
    t_head = time.perf_counter() - t0
    per_token = t_layers * m.n_layers / n_done + t_head
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    threads = min(threads, len(os.sched_getaffinity(0)))
    sample = (f"{n_done} of {m.n_layers} layers ({n_done // 4} [SWA,SWA,SWA,full] blocks at 16,384 cached) "
              f"+ final norm + bf16 lm_head, timed {t_layers + t_head:.1f} s, extrapolated x{m.n_layers / n_done:g} "
              f"over layers")
    out = {"value": 1.0 / per_token, "unit": "tokens/s", "cores": threads, "kind": "oracle", "sample": sample,
           "s_per_token": per_token, "host": host_info()}
    # the same oracle on one thread: one [SWA,SWA,SWA,full] block in a child process
    # started with OMP_NUM_THREADS=1, scaled like the layers above (the head's share
    # scaled by the same thread ratio as the layers)
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-block-seconds", str(config)],
                           env=env, capture_output=True, text=True, timeout=600)
        t1 = float(r.stdout.strip().splitlines()[-1])
        t_multi = t_layers * 4 / n_done
        per_token_1 = t1 * m.n_layers / 4 + t_head * t1 / t_multi
        out["single_thread"] = {"value": 1.0 / per_token_1, "unit": "tokens/s", "cores": 1,
                                "sample": f"one [SWA,SWA,SWA,full] block at 16,384 cached, timed {t1:.1f} s, "
                                          f"extrapolated x{m.n_layers // 4} over layers (head scaled alike)"}
    except (subprocess.SubprocessError, ValueError, IndexError) as e:
        log(f"single-thread oracle leg failed: {e}")
    return out


def oracle_layer_configs(configs=(0, 1, 2), runs=3):
    """Median seconds of one oracle layer step for the single-layer workloads (config 0:
    the tiny layer; 1: a full-size SWA layer at 4,096 keys; 2: a full-size full-attention
    layer at 16,385 keys with YaRN), inputs generated outside the timed region."""
    import statistics
    import oracle as O
    from oracle import runner as R
    from synth import workloads as W
    from swa_attention_amd import accounting as A
    out = {}
    for c in configs:
        wl = W.config(c)
        m = wl.model
        T, Kc, Vc = R.layer_inputs(wl, 0)
        x = W.x_in(m, wl.seed)
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            O.layer_step(m, m.layer_types[0], T, x, Kc, Vc, wl.n_cached)
            ts.append(time.perf_counter() - t0)
        med = statistics.median(ts)
        b = A.decode_step_bytes(m, wl.n_cached, head=False).total
        out[str(c)] = {"workload": wl.name, "us_per_step": round(med * 1e6, 1), "runs": runs,
                       "GBps": round(b / med / 1e9, 3), "bytes_per_step": b}
        del T, Kc, Vc
    return out


def oracle_prefill_baseline(budget_tokens=16):
    """The oracle's prefill (its definition: teacher-forced decode) on the 4-layer
    [SWA, SWA, SWA, full] truncation of the 1,200-token workload, for the first
    budget_tokens tokens; extrapolated linearly over tokens (the weight GEMVs, not the
    attention over <= 1,200 keys, dominate each position) and x16 over layers."""
    import oracle as O
    from oracle import runner as R
    from synth import workloads as W
    pw = W.config(4)
    m = pw.model
    toks = W.prompt_tokens(m, pw.seed, budget_tokens)
    Ts = [W.layer_tensors(m, pw.seed, l) for l in range(4)]
    caches = [W.kv_cache(m, pw.seed, l, 0, budget_tokens) for l in range(4)]
    rows = {int(t): W.embedding_rows(m, pw.seed, int(t), 1)[0] for t in toks}
    t_sum = 0.0
    for t, tok in enumerate(toks):
        x = O.embed(rows[int(tok)])
        t0 = time.perf_counter()
        for l in range(4):
            x = O.layer_step(m, m.layer_types[l], Ts[l], x, caches[l][0], caches[l][1], t)
        t_sum += time.perf_counter() - t0
    ttft_s = t_sum * (pw.prompt_len / budget_tokens) * (m.n_layers / 4)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    threads = min(threads, len(os.sched_getaffinity(0)))
    return {"value": round(pw.prompt_len / ttft_s, 3), "unit": "prompt tokens/s", "ttft_s": round(ttft_s, 1),
            "cores": threads, "kind": "oracle",
            "sample": f"4-layer [SWA,SWA,SWA,full] truncation, first {budget_tokens} of {pw.prompt_len} tokens "
                      f"timed {t_sum:.1f} s; extrapolated x{pw.prompt_len / budget_tokens:g} over tokens and "
                      f"x{m.n_layers // 4} over layers (lm_head not included)"}


def measure_layer_configs(dev, steps=30, copies=3):
    """Decode step of one full-size layer (config 1: SWA at 4,096 keys; config 2: full
    attention at 16,385 keys with YaRN), timed over `copies` independent device copies
    of the layer's weights and KV cache taken in turn, so that a step never finds its
    layer in the ~256 MB memory-side cache left by the previous step. HIP graph of one
    step per copy, replayed."""
    import torch
    from synth import workloads as W
    from synth.device import build_model
    from swa_attention_amd import accounting as A
    from swa_attention_amd import ops
    out = {}
    for c in (1, 2):
        wl = W.config(c)
        m = wl.model
        dms = [build_model(wl, dev) for _ in range(copies)]   # same seeded values at distinct addresses
        cms = [d.c() for d in dms]
        x = torch.from_numpy(W.x_in(m, wl.seed)).to(dev)
        pos = torch.tensor([wl.n_cached], dtype=torch.int32, device=dev)
        ws = torch.empty(ops.atlas_decode_workspace_bytes(dms[0]), dtype=torch.uint8, device=dev)

        def one_round():
            for d, cm in zip(dms, cms):
                ops.atlas_decode_step(d, pos, hidden_in=x, ws=ws, cm=cm)

        one_round()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            one_round()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one_round()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        assert ops.atlas_device_status(ws) == 0
        us = e0.elapsed_time(e1) * 1e3 / (steps * copies)
        b = A.decode_step_bytes(m, wl.n_cached, head=False).total
        out[str(c)] = {"workload": wl.name, "us_per_step": round(us, 2), "GBps": round(b / (us * 1e-6) / 1e9, 1),
                       "frac_of_peak": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4), "bytes_per_step": b,
                       "method": f"{copies} device copies of the layer ({copies} x {b / 1e6:.1f} MB) taken in turn, "
                                 f"HIP graph replays ({steps} x {copies} steps)"}
        log(f"layer config {c}: {us:.1f} us per step, {out[str(c)]['GBps']} GB/s")
        del dms, cms, ws, g
        torch.cuda.empty_cache()
    return out


PEAK_BF16_TFLOPS = 2500.0
PEAK_INT8_TOPS = 5000.0


def measure_prefill(args, dm, cm, m, dev, wl_name):
    """Time-to-first-token of the 1,200-token prompt (same 64-layer model, positions
    0..1,199, written over the decode cache after the decode timing): token ids on
    device to the last row's logits and argmax."""
    import torch
    from synth import workloads as W
    from swa_attention_amd import accounting as A
    from swa_attention_amd import ops
    pw = W.config(4)
    n = pw.prompt_len
    # the prompt runs on the decode workload's model (its weight and KV formats)
    name = pw.name if wl_name == W.config(3).name else wl_name.replace("decode-16k", "prefill-1200").replace(
        "decode-64k", "prefill-1200")
    toks = torch.from_numpy(W.prompt_tokens(m, pw.seed, n)).to(dev)
    ws = torch.empty(ops.atlas_prefill_workspace_bytes(dm, n), dtype=torch.uint8, device=dev)
    logits = torch.empty(m.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)

    def run():
        ops.atlas_prefill(dm, toks, 0, logits, am, ws, cm=cm)

    log(f"prefill {name}: warm-up")
    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.prefill_reps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.prefill_reps
    assert ops.atlas_device_status(ws) == 0
    ops.atlas_profile_start(100000)
    run()
    prof = ops.atlas_profile_stop()
    log("prefill per-launch timing: " + ", ".join(f"{k} {v[0]}x {v[1] / v[0] * 1e3:.1f}us" for k, v in
                                                  sorted(prof.items(), key=lambda kv: -kv[1][1])))
    flops = A.prefill_flops(m, n)
    out = {"workload": name, "tokens": n, "ttft_ms": round(ms, 2), "reps": args.prefill_reps,
           "tokens_per_s": round(n / (ms * 1e-3), 1),
           "algorithmic_tflop": round(flops / 1e12, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "dtype": ("int8 matrix cores for the W4 projections (activations as 24-bit fixed point per row and "
                     "group of 128 in three int8 digit planes, exact int32 sums, f32 accumulation); bf16 matrix "
                     "cores for attention with hi/lo operand planes (about 16 significant bits per product)"),
           "mfma_frac_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    dom = "pf_gemm_gate_up"
    if dom in prof:
        cnt, tot = prof[dom]
        f = 2.0 * n * 2 * m.dff * m.d   # algorithmic flops of one gate+up launch
        ach = f / (tot / cnt * 1e-3) / 1e12
        if m.group % 128 == 0 and m.group <= 512 and m.d % m.group == 0:
            # groups of 128-512: products on the int8 matrix cores, priced at the int8 peak
            out["roofline"] = {"bound": "mfma", "kernel": "w4_gemm_i8r_kernel<1> (gate+up, SwiGLU)",
                               "achieved": round(ach, 1), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                               "frac": round(ach / PEAK_INT8_TOPS, 4), "avg_launch_us": round(tot / cnt * 1e3, 1),
                               "note": "algorithmic multiply-adds x 2; the three int8 digit planes of the "
                                       "activations issue three times as many"}
        else:
            out["roofline"] = {"bound": "mfma", "kernel": "w4_gemm_kernel<1> (gate+up, SwiGLU)",
                               "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(ach / PEAK_BF16_TFLOPS, 4), "avg_launch_us": round(tot / cnt * 1e3, 1),
                               "note": "algorithmic flops; the bf16 hi/lo activation planes issue twice as many"}
    # causal attention of the prompt (positions 0 .. n-1): 4 hd flops per (query, key) pair
    # and query head (QK^T and PV), keys limited to the window on the window layers
    att = {k: prof[k] for k in ("pf_attn_window", "pf_attn_full") if k in prof}
    if att:
        def pairs(window):
            return sum(min(t, window - 1) + 1 for t in range(n)) if window > 0 else n * (n + 1) // 2
        fl = {"pf_attn_window": 4.0 * m.hd * m.hq * pairs(m.window), "pf_attn_full": 4.0 * m.hd * m.hq * pairs(0)}
        cnt = sum(c for c, _ in att.values())
        tot_ms = sum(t for _, t in att.values())
        ach = sum(att[k][0] * fl[k] for k in att) / (tot_ms * 1e-3) / 1e12
        out["attention"] = {"bound": "mfma", "kernel": f"pf_attn_kernel<{m.hq // m.hkv}> (causal GQA)",
                            "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(ach / PEAK_BF16_TFLOPS, 4), "avg_launch_us": round(tot_ms / cnt * 1e3, 1),
                            "launches": cnt,
                            "note": "algorithmic flops; the bf16 hi/lo operand planes issue "
                                    + ("two" if m.kv_dtype == 1 else "three") + " products per multiply-add"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload config (3 = 64-layer 16K decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle compute in the CPU leg")
    ap.add_argument("--profile-steps", type=int, default=3)
    ap.add_argument("--no-prefill", action="store_true", help="skip the 1,200-token prefill measurement")
    ap.add_argument("--prefill-reps", type=int, default=3)
    ap.add_argument("--eager", action="store_true", help="time eager steps instead of HIP graph replays")
    ap.add_argument("--no-sampling", action="store_true", help="skip the on-device sampling measurement")
    ap.add_argument("--no-layer-configs", action="store_true",
                    help="skip the single-layer workloads (full-size SWA and full-attention layers)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode step: no sampling, read probe, layer configs, prefill or CPU legs "
                         "(for profiler runs)")
    ap.add_argument("--stream-probe-gib", type=float, default=2.0,
                    help="buffer size of the plain read-bandwidth probe (0 to skip)")
    ap.add_argument("--oracle-block-seconds", type=int, default=None, help=argparse.SUPPRESS)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (3 times); its HBM counters "
                         "calibrate the FETCH_SIZE/WRITE_SIZE readings of the decode kernels")
    args = ap.parse_args()
    if args.oracle_block_seconds is not None:   # the single-thread oracle leg (a child process)
        print(oracle_block_seconds(args.oracle_block_seconds, 1))
        return
    if args.decode_only:
        args.no_sampling = args.no_layer_configs = args.no_prefill = args.no_cpu_baseline = True
        args.stream_probe_gib = 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "The step would shard by KV head (attention local, two small all-reduces per layer); "
              "only the one-GPU path is built.", file=sys.stderr)
        sys.exit(2)

    import torch
    from synth import workloads as W
    from synth.device import build_model
    from swa_attention_amd import accounting as A
    from swa_attention_amd import ops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wl = W.config(args.config)
    m = wl.model
    log(f"workload {wl.name}: building the device model ({m.n_layers} layers)")
    t0 = time.time()
    dm = build_model(wl, dev, progress=lambda l: (l % 8 == 7) and log(f"  layer {l + 1}/{m.n_layers} resident"))
    torch.cuda.synchronize()
    log(f"model resident in {time.time() - t0:.1f} s, {torch.cuda.memory_allocated() / 1e9:.1f} GB allocated")

    # the seeded first token: the first draw of the workload's prompt stream
    tok = torch.tensor([int(W.prompt_tokens(m, wl.seed, 1)[0])], dtype=torch.int32, device=dev)
    pos = torch.tensor([wl.n_cached], dtype=torch.int32, device=dev)
    head = wl.final_head
    B = wl.batch
    if B > 1:   # batched decode: one token per sequence, every sequence at its own position
        tok = torch.from_numpy(W.batch_tokens(wl)).to(dev)
        pos = torch.tensor([wl.seq_cached(b) for b in range(B)], dtype=torch.int32, device=dev)
    logits = torch.empty((B, m.vocab) if B > 1 else m.vocab, dtype=torch.float32, device=dev) if head else None
    am = tok if head else None      # each step feeds back its argmax
    hidden = torch.empty(m.d, dtype=torch.float32, device=dev)
    x_in = None if wl.use_tokens else torch.from_numpy(W.x_in(m, wl.seed)).to(dev)
    cm = dm.c()
    if B > 1:
        ws = torch.empty(ops.atlas_decode_batch_workspace_bytes(dm, B), dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(ops.atlas_decode_workspace_bytes(dm), dtype=torch.uint8, device=dev)

    def step():
        if B > 1:
            ops.atlas_decode_batch(dm, tok, pos, logits=logits, argmax=am, ws=ws, cm=cm)
        else:
            ops.atlas_decode_step(dm, pos, d_token=tok if wl.use_tokens else None, hidden_in=x_in,
                                  hidden_out=None if head else hidden, logits=logits, argmax=am, ws=ws, cm=cm)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if not args.eager:
        # capture one step (warmed up on the capture stream first); replays run on the
        # current stream like eager steps
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        run = graph.replay
    log(f"timing {args.steps} steps ({'eager' if args.eager else 'HIP graph replays'})")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        run()
        evs[i + 1].record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    pct = lambda q: per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]
    step_ms = {"median": round(pct(0.5), 4), "p10": round(pct(0.1), 4), "p90": round(pct(0.9), 4)}
    assert ops.atlas_device_status(ws) == 0

    # per-launch timing pass: each dispatch stamps a start and a stop hipEvent on its stream
    ops.atlas_profile_start(4096 * max(1, args.profile_steps))
    for _ in range(args.profile_steps):
        step()
    prof = ops.atlas_profile_stop()
    log("per-launch timing: " + ", ".join(f"{k} {v[0]}x {v[1] / v[0] * 1e3:.1f}us" for k, v in
                                          sorted(prof.items(), key=lambda kv: -kv[1][1])))

    if B > 1:
        sb = A.decode_batch_bytes(m, [wl.seq_cached(b) for b in range(B)], head=head)
    else:
        sb = A.decode_step_bytes(m, wl.n_cached, head=head)
    gbps = sb.total / (ms * 1e-3) / 1e9
    dom = "w4_gemv_gate_up" if B == 1 else ("bd_gemv_gate_up" if "bd_gemv_gate_up" in prof else "bd_gemm_gate")
    roof = None
    if dom in prof:
        cnt, tot = prof[dom]
        avg_s = tot / cnt * 1e-3
        # one launch streams the gate and the up matrix ([dff][d] each); the batched GEMM
        # of the bf16-plane path streams the gate matrix alone
        per_launch = (1 if dom == "bd_gemm_gate" else 2) * A.w4_bytes(m.dff, m.d, m.group, 2, not m.symmetric)
        ach = per_launch / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": measured_traffic() if args.config == 3 else None,
                "kernel": (f"gate_up_kernel (2 x {m.dff}x{m.d} W4 + SwiGLU)" if B == 1 else
                           f"bgemv_kernel: gate and up projections of {B} rows (2 x {m.dff}x{m.d} W4, int8 MFMA)"
                           if dom == "bd_gemv_gate_up" else
                           f"gate projection over {B} rows ({m.dff}x{m.d} W4, split over K)"),
                "bytes_per_launch": per_launch,
                "avg_launch_us": round(avg_s * 1e6, 2), "launches": cnt,
                "duration_source": "dispatch-stamped HIP events on the launch stream, eager timing steps"}
        rp = profiled_replay_us() if (args.config == 3 and B == 1) else None
        if rp:   # the committed rocprofv3 trace of the same command, timed graph replays only
            roof["rocprof_graph_replay_avg_us"] = rp
            roof["rocprof_frac"] = round(per_launch / (rp * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)

    sampling = None
    if head and B == 1 and not args.no_sampling:   # the on-device sampler at the card's settings
        wss = torch.empty(ops.atlas_sample_workspace_bytes(m.vocab), dtype=torch.uint8, device=dev)
        du = torch.tensor([0.5], dtype=torch.float32, device=dev)
        tok_s = torch.empty(1, dtype=torch.int32, device=dev)
        for _ in range(3):
            ops.atlas_sample(logits, 0.6, 0.95, du, tok_s, wss)
        torch.cuda.synchronize()
        n_calls = 50
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_calls):
            ops.atlas_sample(logits, 0.6, 0.95, du, tok_s, wss)
        e1.record()
        torch.cuda.synchronize()
        ops.atlas_profile_start(64)
        ops.atlas_sample(logits, 0.6, 0.95, du, tok_s, wss)
        sp = ops.atlas_profile_stop()
        sampling = {"temperature": 0.6, "top_p": 0.95, "vocab": m.vocab,
                    "us_per_call": round(e0.elapsed_time(e1) * 1e3 / n_calls, 2),
                    "kernels_us": {k: round(v[1] / v[0] * 1e3, 2) for k, v in sp.items()},
                    "note": "timed apart from the greedy step above"}
        log(f"sampling: {sampling['us_per_call']} us per call")

    stream = None
    if args.stream_probe_gib > 0:
        nbytes = int(args.stream_probe_gib * 2**30) // 16 * 16
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        best = None
        for blocks in (256, 512, 1024, 2048):
            ops.atlas_stream_read(buf, blocks, sink)
            ops.atlas_profile_start(64)
            for _ in range(5):
                ops.atlas_stream_read(buf, blocks, sink)
            cnt, tot = ops.atlas_profile_stop()["stream_read"]
            g = nbytes / (tot / cnt * 1e-3) / 1e9
            if best is None or g > best[0]:
                best = (g, blocks)
        del buf, sink
        stream = {"GBps": round(best[0], 1), "frac_of_peak": round(best[0] / PEAK_HBM_GBPS, 4), "bytes": nbytes,
                  "blocks": best[1], "kernel": "stream_read_kernel (plain grid-stride read, 4 x 16 B in flight "
                                               "per thread; best of 256-2,048 blocks)"}
        log(f"plain read probe: {best[0]:.0f} GB/s with {best[1]} blocks")

    prefill = None
    if not args.no_prefill and head and wl.use_tokens and B == 1:
        prefill = measure_prefill(args, dm, cm, m, dev, wl.name)

    layer_cfgs = None
    if not args.no_layer_configs and args.config == 3:
        layer_cfgs = measure_layer_configs(dev)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 18   # f32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 3 x {args.copy_probe_mib} MiB device copies")
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline (bounded sample)")
        cpu = cpu_baseline(wl, args.cpu_budget, args.config)
        if args.config == 3:
            log("CPU oracle: single-layer configurations (median of 3)")
            cpu["layer_configs"] = oracle_layer_configs()
            if prefill is not None:
                log("CPU oracle: prefill on the 4-layer truncation (bounded sample)")
                prefill["cpu_baseline"] = oracle_prefill_baseline()

    out = {
        "metric": ("decode tokens/s at batch 1, 32B W4, 16K ctx + achieved HBM GB/s vs peak" if B == 1 else
                   f"aggregate decode tokens/s at batch {B} (tokens of all sequences per second), 32B W4, "
                   f"{wl.n_cached} ctx"),
        "value": round(B * 1e3 / ms, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": step_ms,
        "timing": "eager steps" if args.eager else "HIP graph replays of one captured step",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_detail": (
            "W4 projections: activations as 24-bit block fixed point per 32 columns, exact integer dot "
            "products with the 4-bit codes, f32 accumulation; attention, norms and the bf16 lm_head in f32"
            if B == 1 else
            "W4 projections: activations as 24-bit block fixed point per 128 columns in three int8 digit "
            "planes on the int8 matrix cores (exact int32 digit sums), f32 accumulation; attention and norms "
            "in f32; bf16 lm_head with activations as bf16 hi/lo planes" if B <= 8 else
            "W4 projections on bf16 matrix cores with activations as bf16 hi/lo planes (16 significant bits)"),
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": m.n_layers, "context": wl.n_cached, "batch": B,
                   "weights": (f"int4 group-{m.group}, {'bf16' if m.scale_dtype else 'f16'} scales, "
                               + ("symmetric (zero point 8)" if m.symmetric else "uint4 zeros")),
                   "kv": ("bf16" if m.kv_dtype == 1 else "f32") + (
                       f", ring of {m.window} slots on the sliding-window layers" if m.swa_ring else ""),
                   "lm_head": "bf16"},
        "achieved_GBps": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
        "bytes_per_step": sb.total,
        "roofline": roof,
        "achievable_read": stream,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "layer_configs": layer_cfgs,
        "sampling": sampling,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
