"""Benchmark of the single-token Llama-2 decode step on one MI355X.

Workload (default): the Llama-2-7B-shaped model (dim 4096, hidden 11008, 32
layers, 32 query / 32 kv heads, vocab 32000, seq_len 2048, fp32, seeded random
weights), greedy decode from token 1 at position 0.  One step = one decode
token: every kernel of the path (q/k/v + RoPE + cache append, attention, wo +
residual, w1/w3 SwiGLU, w2 + residual per layer; classifier + argmax) runs
once.  The weights are resident in HBM before the timed region starts.

Output: one JSON line with decode tokens/s, achieved HBM GB/s (algorithmic
bytes read per token / time), the roofline of the dominant kernel (its average
launch duration measured with HIP events on the library's stream over a pass
of the same workload; for the GEMV kernels the events are recorded by the
kernel's own dispatch), the practical read ceiling (a plain streaming read
timed just before the decode), the next rows' legs and the CPU oracle timed on
a bounded sample.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]
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

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix


def prefill_flops(c, n: int) -> int:
    """Algorithmic flops of a prefill of n tokens from position 0: 2 per weight
    of every layer projection per token, 4 per head dimension per (query, key)
    pair of the causal attention (scores and the weighted sum), and the
    classifier for the last token."""
    kv = c.dim * c.n_kv_heads // c.n_heads
    proj = 2 * c.dim * c.dim + 2 * kv * c.dim + 3 * c.dim * c.hidden_dim
    pairs = n * (n + 1) // 2
    return 2 * c.n_layers * proj * n + 4 * c.n_layers * c.dim * pairs + 2 * c.vocab_size * c.dim


def bytes_per_token(c, pos: int) -> int:
    """Algorithmic bytes read by one decode step at position pos: every weight
    once (layer matrices and gains, the whole classifier, one embedding row, the
    final gain) plus the key and value rows 0..pos of every layer."""
    kv = c.dim * c.n_kv_heads // c.n_heads
    per_layer = 2 * c.dim * c.dim + 2 * kv * c.dim + 3 * c.dim * c.hidden_dim + 2 * c.dim
    floats = c.n_layers * per_layer + c.vocab_size * c.dim + 2 * c.dim
    return 4 * floats + 4 * 2 * c.n_layers * (pos + 1) * kv


def kernel_bytes(c, kind: str, pos_list) -> float:
    """Algorithmic bytes moved per launch of one kernel kind, averaged over the
    positions of the pass (only attention depends on the position)."""
    d, h, V = c.dim, c.hidden_dim, c.vocab_size
    kv = d * c.n_kv_heads // c.n_heads
    if kind == "qkv_rope_append":  # Wq, Wk, Wv + x + gain; q and the cache row written
        return 4.0 * ((d + 2 * kv) * d + 2 * d + d + 2 * kv)
    if kind == "wo_residual":  # Wo + xb + x read and written
        return 4.0 * (d * d + d + 2 * d)
    if kind == "w1w3_swiglu":  # W1, W3 + x + gain; hb written
        return 4.0 * (2 * h * d + 2 * d + h)
    if kind == "w2_residual":  # W2 + hb + x read and written
        return 4.0 * (d * h + h + 2 * d)
    if kind == "classifier_argmax":  # Wcls + x + gain; logits written
        return 4.0 * (V * d + 2 * d + V)
    if kind == "qkv_attention":  # the q/k/v product (q handed over on chip) and the attention: Wq, Wk, Wv + x +
        # gain, the cache row written, key and value rows 0..pos-1 read, output
        mean_rows = sum(p for p in pos_list) / len(pos_list)
        return 4.0 * ((d + 2 * kv) * d + 2 * d + 2 * kv + 2 * kv * mean_rows + d)
    if kind == "attention":  # q, key and value rows 0..pos of one layer, output
        mean_rows = sum(p + 1 for p in pos_list) / len(pos_list)
        return 4.0 * (2 * d + 2 * kv * mean_rows)
    raise KeyError(kind)


def source_digest() -> str:
    h = hashlib.sha256()
    for name in ("ld_kernels.hip", "ld_runtime.hip", "ld_internal.h"):
        with open(os.path.join(ROOT, "llama_transformer_decode_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != source_digest():
        return None
    return t.get("bytes_per_launch")


# Where each workload's timed decode starts: the 70B-layer workload first fills
# the cache with 3584 seeded tokens through forward calls (untimed), then times
# greedy decode from position 3584 to the end of its 4096-position context.
START = {"llama70b_8l": 3584}


def windows_for(seq_len: int, start: int = 0, width: int = 16):
    """16-step windows whose rates are reported on their own, whatever the
    timed step count: the first positions of the decode, positions 504-519
    (around the 512th token) where the context reaches them, and the last 16
    positions of the context."""
    marks = {start, seq_len - width}
    if start <= 504 and 520 <= seq_len:
        marks.add(504)
    return [(a, min(a + width, seq_len)) for a in sorted(m for m in marks if start <= m < seq_len)]


def median(xs):
    ys = sorted(xs)
    k = len(ys)
    return ys[k // 2] if k % 2 else 0.5 * (ys[k // 2 - 1] + ys[k // 2])


def fill_cache(model, cfg, start: int) -> int:
    """Reset the cache and fill rows 0..start-1 (the 70B-layer workload's seeded
    prompt, through forward calls); returns the first token to decode."""
    import synth
    model.reset()
    if not start:
        return 1
    prompt = synth.prefill_tokens(cfg, start)
    for p in range(start):
        model.forward_async(int(prompt[p]), p)
    return model.argmax_last()


def timed_generations(model, tok: int, pos: int, n: int, reps: int, torch):
    """reps timed greedy generations of n steps from (tok, pos).  Generation is
    deterministic, so every repeat rewrites the same cache rows with the same
    values and takes the same tokens.  Returns (tokens, seconds per repeat)."""
    times, toks = [], None
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks = model.generate(tok, pos, n)
        times.append(time.perf_counter() - t0)
    return toks, times


def kernel_table(cfg, stats, pos_list):
    out = {}
    for s in stats:
        if s["launches"]:
            avg_ms = s["total_ms"] / s["launches"]
            byt = kernel_bytes(cfg, s["name"], pos_list)
            out[s["name"]] = {"launches": s["launches"], "avg_us": round(avg_ms * 1e3, 2),
                              "bytes_per_launch": int(byt), "GBps": round(byt / (avg_ms * 1e-3) / 1e9, 1),
                              "share_of_time": round(s["total_ms"], 3)}
    tot = sum(k["share_of_time"] for k in out.values()) or 1.0
    for k in out.values():
        k["share_of_time"] = round(k["share_of_time"] / tot, 4)
    return out


def decode_legs(model, cfg, start: int, steps: int, reps: int, torch, kernel_timing: bool = True,
                windows: bool = True):
    """The timed decode of one workload on a model whose weights are resident:
    `steps` greedy steps from `start` (the first token after the cache fill),
    timed `reps` times (the median is the value); the per-position windows,
    each timed `reps` times after decoding up to it untimed; and the kernel
    durations of the timed positions and of each window.  Returns a dict."""
    S = cfg.seq_len
    t_fill = time.time()
    first_tok = fill_cache(model, cfg, start)
    torch.cuda.synchronize()
    if start:
        print(f"# {cfg.name}: cache filled by {start} forward calls in {time.time() - t_fill:.1f} s", file=sys.stderr,
              flush=True)
    span = S - start
    passes = [span] * (steps // span) + ([steps % span] if steps % span else [])
    rep_times = []
    for _ in range(reps):
        t_rep = 0.0
        for i, n_pass in enumerate(passes):
            if i:  # more steps than positions: a fresh pass over the context (untimed refill)
                fill_cache(model, cfg, start)
            _, dts = timed_generations(model, first_tok, start, n_pass, 1, torch)
            t_rep += dts[0]
        rep_times.append(t_rep)
    if len(passes) > 1:
        fill_cache(model, cfg, start)
    t_med = median(rep_times)
    print(f"# {cfg.name}: {reps} x {steps} timed steps, median {steps / t_med:.1f} tok/s", file=sys.stderr, flush=True)
    pos_all = [start + (i % span) for i in range(steps)]
    total_bytes = sum(bytes_per_token(cfg, p) for p in pos_all)
    out = {"steps": steps, "positions": [start, start + min(steps, span) - 1], "repeats": reps,
           "seconds": [round(t, 6) for t in rep_times], "tok_s": round(steps / t_med, 2),
           "tok_s_min": round(steps / max(rep_times), 2), "tok_s_max": round(steps / min(rep_times), 2),
           "ms_per_step": round(1e3 * t_med / steps, 4), "hbm_GBps": round(total_bytes / t_med / 1e9, 1)}
    out["hbm_frac_of_peak"] = round(out["hbm_GBps"] / HBM_PEAK_GBPS, 4)

    # per-position windows, decoding through the gaps untimed
    per_pos, win_kernels = {}, {}
    tok, pos = first_tok, start
    for a, b in (windows_for(S, start) if windows else []):
        if pos < a:
            tok = int(model.generate(tok, pos, a - pos)[-1])
            pos = a
        toks, dts = timed_generations(model, tok, a, b - a, reps, torch)
        dt = median(dts)
        byt = sum(bytes_per_token(cfg, p) for p in range(a, b))
        key = f"pos_{a}_{b - 1}"
        per_pos[key] = {"tok_s": round((b - a) / dt, 2), "GBps": round(byt / dt / 1e9, 1),
                        "frac_of_peak": round(byt / dt / 1e9 / HBM_PEAK_GBPS, 4),
                        "tok_s_min": round((b - a) / max(dts), 2), "tok_s_max": round((b - a) / min(dts), 2)}
        if kernel_timing:  # the same positions once more, every launch timed (deterministic: same rows)
            ks = kernel_table(cfg, model.profile(tok, a, b - a), list(range(a, b)))
            win_kernels[key] = {k: v["avg_us"] for k, v in ks.items()}
        tok, pos = int(toks[-1]), b
    out["per_position"] = per_pos
    if win_kernels:
        out["kernels_by_window_us"] = win_kernels

    # kernel durations over the value's positions, every launch timed with HIP events
    if kernel_timing:  # rows start.. are rewritten with the values they hold
        n_prof = min(steps, span)
        out["kernels"] = kernel_table(cfg, model.profile(first_tok, start, n_prof), list(range(start, start + n_prof)))
    out["first_token"] = first_tok
    return out


def read_ceiling(pkg, torch):
    """The practical read ceiling: a plain streaming read of a 4 GiB buffer,
    the best of 3 rounds of 10 reads, timed with HIP events."""
    nbytes = 4 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0")
    sums = torch.empty(pkg.ld.LD_STREAM_READ_BLOCKS, dtype=torch.float32, device="cuda:0")
    st = torch.cuda.current_stream()
    for _ in range(3):
        pkg.ld.ld_op_stream_read(buf.data_ptr(), nbytes, sums.data_ptr(), st.cuda_stream)
    reps, dts = 10, []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            pkg.ld.ld_op_stream_read(buf.data_ptr(), nbytes, sums.data_ptr(), st.cuda_stream)
        e1.record(st)
        torch.cuda.synchronize()
        dts.append(e0.elapsed_time(e1) * 1e-3 / reps)
    dt = min(dts)
    c_gbps = nbytes / dt / 1e9
    del buf, sums
    torch.cuda.empty_cache()
    out = {"kernel": "stream_read_kernel", "bytes_per_launch": nbytes, "avg_us": round(dt * 1e6, 1),
           "GBps": round(c_gbps, 1), "frac_of_peak": round(c_gbps / HBM_PEAK_GBPS, 4)}
    print(f"# read ceiling: {json.dumps(out)}", file=sys.stderr, flush=True)
    return out


def roofline_of(kernels, cfg):
    dom = max(kernels, key=lambda k: kernels[k]["share_of_time"])
    kd = kernels[dom]
    return {"bound": "hbm", "kernel": dom, "achieved": kd["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(kd["GBps"] / HBM_PEAK_GBPS, 4), "traffic": load_traffic(dom, cfg.name),
            "bytes_per_launch": kd["bytes_per_launch"], "avg_us": kd["avg_us"]}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed decode steps (default: seq_len)")
    ap.add_argument("--warmup", type=int, default=32, help="untimed decode steps before the timed pass")
    ap.add_argument("--config", default="llama7b", help="workload: tiny, stories15m, gqa_small, llama7b, llama70b_8l")
    ap.add_argument("--no-graph", action="store_true", help="launch kernels directly instead of graph replay")
    ap.add_argument("--no-fuse", action="store_true",
                    help="launch every layer's attention on its own, also at short contexts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the plain streaming read that measures the practical HBM read ceiling")
    ap.add_argument("--cpu-positions", default=None,
                    help="comma-separated positions of the oracle decode steps timed for the CPU baseline "
                         "(default: the first timed position, 511 and the last one; about 10 s on the 7B shape)")
    ap.add_argument("--prefill-tokens", type=int, default=None,
                    help="prompt length of the timed batched prefill (default: the workload's prompt, else 2048; "
                         "0: skip)")
    ap.add_argument("--batch-sizes", default="1,4,16,64",
                    help="comma-separated batch sizes of the timed batch-decode leg ('' to skip)")
    ap.add_argument("--sampled-steps", type=int, default=256,
                    help="steps of the temperature / top-p generation loop timed beside greedy decode (0: skip)")
    ap.add_argument("--no-windows", action="store_true",
                    help="skip the per-position windows (which decode the whole context): for profiler runs")
    ap.add_argument("--repeats", type=int, default=5,
                    help="times the timed decode and each per-position window are run; the median is reported")
    ap.add_argument("--long-context", default=None,
                    help="second workload timed after the first (default: the 70B-layer workload after the 7B-shaped "
                         "one, none otherwise; 'none' to skip): its cache fill, then its timed decode, windows and "
                         "kernel durations")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB mebibytes three times (reference for "
                         "scaling the HBM byte counters of a profiler) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode step is not sharded across GPUs in this build", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import llama_transformer_decode_amd as pkg
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))
        return 0
    cfg = synth.CONFIGS[args.config]
    S = cfg.seq_len
    start = START.get(cfg.name, 0)
    steps = args.steps or (S - start)
    warm = max(0, args.warmup)

    t = time.time()
    blob = synth.make_blob(cfg)
    t_gen = time.time() - t
    t = time.time()
    weights = torch.from_numpy(blob).to("cuda:0")
    torch.cuda.synchronize()
    t_up = time.time() - t
    print(f"# {cfg.name}: {blob.nbytes / 1e9:.2f} GB of weights generated in {t_gen:.1f} s, uploaded in {t_up:.1f} s",
          file=sys.stderr, flush=True)

    model = pkg.Model(cfg, weights, graph=not args.no_graph, fuse=not args.no_fuse)
    # warm-up: instantiates the per-token graph and touches every kernel
    if warm:
        model.generate(1, 0, min(warm, S))
    torch.cuda.synchronize()

    ceiling = read_ceiling(pkg, torch) if not args.no_read_ceiling else None

    # ---- timed region: `steps` greedy decode steps, `repeats` times; windows; kernel durations ----
    leg = decode_legs(model, cfg, start, steps, args.repeats, torch, kernel_timing=not args.no_kernel_timing,
                      windows=not args.no_windows)
    first_tok = leg["first_token"]
    tok_s, gbps = leg["tok_s"], leg["hbm_GBps"]
    t_total = steps / tok_s
    per_pos = leg["per_position"]
    print(f"# timed {steps} steps x {args.repeats}: median {tok_s:.1f} tok/s "
          f"({leg['tok_s_min']:.1f}-{leg['tok_s_max']:.1f}), {gbps:.0f} GB/s; windows {json.dumps(per_pos)}",
          file=sys.stderr, flush=True)
    kernels = leg.get("kernels")
    roofline = roofline_of(kernels, cfg) if kernels else None
    if kernels:
        print(f"# kernels: {json.dumps(kernels)}", file=sys.stderr, flush=True)
        print(f"# kernels by window (us): {json.dumps(leg.get('kernels_by_window_us'))}", file=sys.stderr, flush=True)

    # ---- the sampling generation loop beside greedy decode, same positions ----
    sampled = None
    if args.sampled_steps > 0:
        n_s = min(args.sampled_steps, S - start)
        coins = synth.coins(n_s, cfg.seed, 7)
        sampled = {"steps": n_s, "positions": [start, start + n_s - 1], "modes": {}}
        for name, T, topp in (("greedy", 0.0, 0.0), ("temperature_0.9", 0.9, 0.0), ("top_p_0.9", 0.9, 0.9)):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            got = model.generate_sampled([first_tok], start, n_s, T, topp, -1, coins)
            dt = time.perf_counter() - t0
            assert got.size == n_s
            sampled["modes"][name] = {"temperature": T, "topp": topp, "tok_s": round(n_s / dt, 2),
                                      "ms_per_step": round(1e3 * dt / n_s, 4)}
        g = sampled["modes"]["greedy"]["ms_per_step"]
        for v in sampled["modes"].values():
            v["us_over_greedy"] = round(1e3 * (v["ms_per_step"] - g), 2)
        print(f"# generation loop: {json.dumps(sampled)}", file=sys.stderr, flush=True)

    # ---- batched prompt prefill on the matrix cores (overwrites the cache) ----
    prefill = None
    n_pf = args.prefill_tokens if args.prefill_tokens is not None else (start or min(S, 2048))
    if n_pf > 0:
        n_pf = min(n_pf, S)
        ptoks = synth.prefill_tokens(cfg, n_pf).copy()
        ptoks[0] = 1
        times = []
        for _ in range(3):
            model.reset()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            model.prefill_async(ptoks, 0)
            model.argmax_last()  # synchronises the stream
            times.append(time.perf_counter() - t0)
        dt = min(times)
        fl = prefill_flops(cfg, n_pf)
        tf = fl / dt / 1e12
        prefill = {"tokens": n_pf, "ms": round(1e3 * dt, 2), "tok_s": round(n_pf / dt, 1),
                   "flops": fl, "TFLOPs": round(tf, 1),
                   "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": FP32_MFMA_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4)},
                   "vs_token_by_token": round((n_pf / dt) / tok_s, 1)}
        print(f"# prefill: {json.dumps(prefill)}", file=sys.stderr, flush=True)

    model.close()

    # ---- batch decode: several sequences per step, each with its own cache ----
    batch = None
    sizes = [int(x) for x in args.batch_sizes.split(",") if x.strip()]
    if sizes:
        n_b = 32
        bpos = min(start, S - n_b - 4)
        batch = {"steps": n_b, "positions": [bpos, bpos + n_b - 1], "sizes": {}}
        with pkg.Model(cfg, weights, max_batch=max(sizes)) as bm:
            for B in sizes:
                starts = synth.prefill_tokens(cfg, B)
                bm.generate_batch(starts, [bpos] * B, 4)  # captures this size's graph
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                bm.generate_batch(starts, [bpos] * B, n_b)
                dt = time.perf_counter() - t0
                kv = cfg.dim * cfg.n_kv_heads // cfg.n_heads
                step_bytes = sum(bytes_per_token(cfg, p) + (B - 1) * 8 * cfg.n_layers * (p + 1) * kv
                                 for p in range(bpos, bpos + n_b))
                batch["sizes"][str(B)] = {"tok_s": round(B * n_b / dt, 1), "ms_per_step": round(1e3 * dt / n_b, 3),
                                          "GBps": round(step_bytes / dt / 1e9, 1)}
        print(f"# batch decode: {json.dumps(batch)}", file=sys.stderr, flush=True)

    del weights
    torch.cuda.empty_cache()

    # ---- CPU baseline: the oracle on a bounded sample of the same workload ----
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cache = oracle.KVCache(cfg)
        if args.cpu_positions:
            cpu_pos = sorted({int(x) for x in args.cpu_positions.split(",") if x.strip()})
        else:
            cpu_pos = sorted({start, S - 1} | ({511} if start <= 511 < S else set()))
        if not cpu_pos or cpu_pos[0] < 0 or cpu_pos[-1] >= S:
            print(f"CPU baseline positions must lie in [0, {S})", file=sys.stderr)
            return 2
        # one thread, pinned to one core; a step's cost does not depend on the
        # cache contents, so each position runs on the zero cache
        allowed = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(allowed)})
        per_step = {}
        for p in cpu_pos:
            t0 = time.perf_counter()
            oracle.forward(cfg, blob, cache, 1, p)
            per_step[str(p)] = time.perf_counter() - t0
        dt = sum(per_step.values())
        per_step = {k: float(f"{v:.4g}") for k, v in per_step.items()}
        n_cpu = len(cpu_pos)
        os.sched_setaffinity(0, allowed)
        cpu_model = ""
        try:
            for ln in open("/proc/cpuinfo"):
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        cpu = {"value": round(n_cpu / dt, 5), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n_cpu} decode steps of the {cfg.name} workload at positions "
                         f"{', '.join(map(str, cpu_pos))} (zero cache), single-threaded C oracle with double "
                         f"accumulation, {dt:.1f} s",
               "seconds_per_step": per_step,
               "GBps": round(sum(bytes_per_token(cfg, p) for p in cpu_pos) / dt / 1e9, 2),
               "host_cores_available": os.cpu_count(), "pinned_core": min(allowed), "cpu_model": cpu_model}
        # the same sample with the rows of every matrix-vector product (and the
        # heads of every attention call) shared out over the host's cores in
        # contiguous ranges, the row-parallel matmul of the "run.c" page; the
        # results are bit-identical to one thread's
        n_thr = max(1, min(len(allowed), 16))
        oracle.set_threads(n_thr)
        try:
            per_mt = {}
            for p in cpu_pos:
                t0 = time.perf_counter()
                oracle.forward(cfg, blob, cache, 1, p)
                per_mt[str(p)] = time.perf_counter() - t0
        finally:
            oracle.set_threads(1)
        dt_mt = sum(per_mt.values())
        cpu["all_cores"] = {"value": round(n_cpu / dt_mt, 5), "unit": "tokens/s", "cores": n_thr,
                            "seconds_per_step": {k: float(f"{v:.4g}") for k, v in per_mt.items()},
                            "GBps": round(sum(bytes_per_token(cfg, p) for p in cpu_pos) / dt_mt / 1e9, 2)}

    # ---- the long-context workload: the 70B-layer model, decode from 3584 to 4095 ----
    long_ctx = None
    lc_name = args.long_context or ("llama70b_8l" if cfg.name == "llama7b" else "none")
    if lc_name != "none":
        del blob
        lcfg = synth.CONFIGS[lc_name]
        lstart = START.get(lcfg.name, 0)
        t = time.time()
        lblob = synth.make_blob(lcfg)
        lweights = torch.from_numpy(lblob).to("cuda:0")
        del lblob
        torch.cuda.synchronize()
        print(f"# {lcfg.name}: weights generated and uploaded in {time.time() - t:.1f} s", file=sys.stderr, flush=True)
        with pkg.Model(lcfg, lweights, graph=not args.no_graph, fuse=not args.no_fuse) as lm:
            if warm:
                lm.generate(1, 0, min(warm, lcfg.seq_len))
            t = time.time()
            lsteps = lcfg.seq_len - lstart
            lleg = decode_legs(lm, lcfg, lstart, lsteps, args.repeats, torch,
                               kernel_timing=not args.no_kernel_timing, windows=not args.no_windows)
        del lweights
        torch.cuda.empty_cache()
        long_ctx = {"workload": f"{lcfg.name}: {lstart} seeded prompt tokens through forward calls (untimed), "
                                f"then greedy decode of positions {lstart}-{lcfg.seq_len - 1}, batch 1, dim {lcfg.dim}, "
                                f"hidden {lcfg.hidden_dim}, {lcfg.n_layers} layers, {lcfg.n_heads}/{lcfg.n_kv_heads} "
                                f"heads, vocab {lcfg.vocab_size}, fp32 N(0,0.02) weights (seed {lcfg.seed})"}
        long_ctx.update({k: v for k, v in lleg.items() if k != "first_token"})
        if lleg.get("kernels"):
            long_ctx["roofline"] = roofline_of(lleg["kernels"], lcfg)
        print(f"# long context: {json.dumps(long_ctx)}", file=sys.stderr, flush=True)

    if ceiling:
        ceiling["decode_frac_of_ceiling"] = round(gbps / ceiling["GBps"], 4)
        if roofline:
            ceiling["dominant_kernel_frac_of_ceiling"] = round(roofline["achieved"] / ceiling["GBps"], 4)

    line = {
        "metric": "batch-1 decode tokens/sec + achieved HBM GB/s as % of MI355X peak",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": leg["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: greedy decode of {steps} tokens from position {start}"
                               f"{' after a ' + str(start) + '-token seeded prefill' if start else ' (token 1)'}, batch 1, "
                               f"dim {cfg.dim}, hidden {cfg.hidden_dim}, {cfg.n_layers} layers, "
                               f"{cfg.n_heads}/{cfg.n_kv_heads} heads, vocab {cfg.vocab_size}, "
                               f"seq_len {cfg.seq_len}, fp32 N(0,0.02) weights (seed {cfg.seed})",
                   "global_batch": 1, "seq_len": cfg.seq_len, "parallelism": "single-gpu",
                   "graph_replay": not args.no_graph},
        "hbm_GBps": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_token_pos0": bytes_per_token(cfg, 0),
        "repeats": {"n": args.repeats, "seconds": leg["seconds"], "tok_s_min": leg["tok_s_min"],
                    "tok_s_max": leg["tok_s_max"]},
        "per_position": per_pos,
        "roofline": roofline,
        "kernels": kernels,
        "kernels_by_window_us": leg.get("kernels_by_window_us"),
        "generation_loop": sampled,
        "prefill": prefill,
        "batch_decode": batch,
        "long_context": long_ctx,
        "read_ceiling": ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
