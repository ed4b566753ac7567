#!/usr/bin/env python3
"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

Headline step (the `value`): one decode-attention call over a packed K4/V2
cache -- batch 16, 28 query heads over 4 kv heads, d=128, 32768 tokens, fp16
queries -- i.e. query prep + split-K scan + combine/inverse transform.  The
timed steps rotate over 4 replicas of the 210 MB cache (a decode step reads a
different layer's cache each time), so the 256 MB Infinity Cache cannot serve
them.  `value` is algorithmic bytes per step (packed cache + queries + output)
divided by the step time.

The decode leg also times the same step with a 128-token fp16 residual window
per sequence (tq_attn_decode_rw).  Further legs in the same JSON line:
tq_encode throughput (4 kv heads x 8192
tokens, fp16, K 4-bit + V 2-bit per step, over a 1 GiB rotating input pool),
long-context decode (8 kv heads x 2^20 tokens, K3/V3, 64 bf16 query heads) and
inner-product search (2^20 x 256 database, 3-bit + QJL m=256, 1024 queries,
top-10; useful estimator TFLOP/s, and the matrix-core work issued against the
dense fp16 peak), and decode over the caches of the rotation / norm variants
(head_dim 64 with the double transform on the scan; head_dim 512 with one norm
per 256-half on the vector-ALU kernel).  `roofline` is the scan kernel's algorithmic bytes per launch over its
mean launch time, measured with HIP events recorded on the launch stream around
the scan launch of every timed step (so the scan time is part of, and never
longer than, the step time); `traffic` is the HBM bytes per scan launch from the
committed FETCH_SIZE / WRITE_SIZE summary under profiles/ (null once the scan
sources differ from the ones measured).  `read_ceiling` is the library's
read-only streaming kernel (tq_stream_read: 16-byte loads over 1 GiB, beyond
the 256 MB Infinity Cache) timed the same way.
`cpu_baseline` is the CPU oracle timed on bounded samples of the workloads
(decode, encode, tiny, search, long context).  Inputs are synthetic and seeded
(synth.py).

The default warmup (2000 untimed steps, about 0.15 s of back-to-back decode) lets
the GPU reach its sustained clock: a decode loop run straight from idle is
timed while the clocks still ramp, which reads about 20% slower than the steady
state a serving loop runs in.

With --power the decode leg also samples board power and GFX clock (amd-smi)
while the scan alone, and then a read-only stream, run back to back, after a
reading of the idle board ("power" under "decode").

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs decode,encode,long,search,variants,quality]
                       [--power]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_scan_traffic_b16_h28x4_ctx32768_k4v2.txt")
# sources of the scan kernel: a stored traffic measurement is used only while these are unchanged
SCAN_SOURCES = ("kv_cache_vector_02_amd/csrc/tq_attn_kernels.h", "kv_cache_vector_02_amd/csrc/tq_attn.hip",
                "kv_cache_vector_02_amd/csrc/tq_device.h", "kv_cache_vector_02_amd/csrc/tq_internal.h")
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix cores, published
PROBE_EVERY = 8                 # timed steps between two carrying kernel-timing events

METRIC = "packed-KV decode attn GB/s & % HBM peak (1 GPU); tq_encode Mvectors/s"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--legs", default="decode,encode,long,search,variants,quality")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--power", action="store_true",
                    help="decode leg: board power and GFX clock (amd-smi) while the scan, and then a read-only "
                         "stream, run back to back; idle power first")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration for --pmc runs)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def scan_source_hash():
    import hashlib

    h = hashlib.sha256()
    for rel in SCAN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per scan launch from the committed FETCH_SIZE / WRITE_SIZE
    summary, each counter scaled by its reading on a copy of known size; None
    when the summary is missing or the kernel sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv.get("scan_source_sha256") != scan_source_hash():
            return None
        fetch = float(kv["fetch_kib_per_dispatch"]) * 1024 * float(kv["fetch_scale"])
        write = float(kv["write_kib_per_dispatch"]) * 1024 * float(kv["write_scale"])
    except (KeyError, ValueError, OSError):
        return None
    return {"bytes": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
            "source": os.path.relpath(TRAFFIC_FILE, ROOT)}


def timed_loop(fn, steps, warmup, torch, probe=False):
    """Runs fn(i, ev) for warmup + steps iterations; returns ms per timed step.

    With probe=True every PROBE_EVERY-th timed step (from the first) gets a
    pair of timing events `ev` that fn records around the kernel it wants timed
    (on the launch stream, which is torch's current stream); the mean probed
    duration is returned as well.  Event markers between the launches of every
    step would add about 8 us per 55 us decode step on MI355X, so only a sample
    of the steps carries them."""
    for i in range(warmup):
        fn(i, None)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           if probe and i % PROBE_EVERY == 0 else None for i in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        fn(warmup + i, evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    if not probe:
        return ms
    probed = [a.elapsed_time(b) for a, b in (e for e in evs if e is not None)]
    return ms, sum(probed) / len(probed)


def attn_step(tq, args, ev):
    """One decode step as its three launches; the scan between the events."""
    tq.tq_attn_prepare(*args)
    if ev is not None:
        ev[0].record()
    tq.tq_attn_scan(*args)
    if ev is not None:
        ev[1].record()
    tq.tq_attn_combine(*args)


def _smi_sample():
    """One amd-smi reading: board power (W) and the mean GFX clock (MHz) of GPU 0."""
    import re
    import subprocess

    r = subprocess.run(["amd-smi", "metric", "-p", "-c", "-g", "0"], capture_output=True, text=True, timeout=20)
    pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", r.stdout)
    clk = [float(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", r.stdout)]
    return (float(pw.group(1)) if pw else None), (sum(clk) / len(clk) if clk else None)


def power_probe(fn, seconds, torch):
    """Runs fn(i) back to back for about `seconds` while a thread samples
    amd-smi; the first third of the samples (clock and power ramp) is dropped.
    fn=None samples the idle board."""
    import threading
    import time

    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                samples.append(_smi_sample())
            except Exception:  # noqa: BLE001 -- a failed reading is skipped
                pass
            time.sleep(0.25)

    torch.cuda.synchronize()
    th = threading.Thread(target=sampler)
    th.start()
    n, t0 = 0, time.time()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    while time.time() - t0 < seconds:
        if fn is None:
            time.sleep(0.1)
            continue
        for _ in range(100):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    b.record()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    steady = samples[len(samples) // 3:]
    pw = [p for p, _ in steady if p is not None]
    ck = [c for _, c in steady if c is not None]
    out = {"samples": len(steady), "power_w": sum(pw) / len(pw) if pw else None,
           "power_w_max": max(pw) if pw else None, "gfx_mhz": sum(ck) / len(ck) if ck else None}
    if fn is not None:
        out["launches"] = n
        out["ms_per_launch"] = a.elapsed_time(b) / n
        if pw:
            out["energy_mj_per_launch"] = out["power_w"] * out["ms_per_launch"]
    return out


# ------------------------------------------------------------------ decode ----
def decode_leg(tq, torch, synth, steps, warmup, replicas=4, power=False):
    B, Hkv, g, ctx, d, kb, vb = 16, 4, 7, 32768, 128, 4, 2
    Hq = Hkv * g
    kc, vc = tq.tq_codebook(kb, d, 42), tq.tq_codebook(vb, d, 42)
    K, V = synth.decode_cache_inputs(B, Hkv, ctx, d, device="cuda")
    caches = []
    for _ in range(replicas):
        c = {
            "k_codes": torch.empty(B, Hkv, ctx, kc.code_bytes, dtype=torch.uint8, device="cuda"),
            "k_norms": torch.empty(B, Hkv, ctx, dtype=torch.float16, device="cuda"),
            "v_codes": torch.empty(B, Hkv, ctx, vc.code_bytes, dtype=torch.uint8, device="cuda"),
            "v_norms": torch.empty(B, Hkv, ctx, dtype=torch.float16, device="cuda"),
        }
        tq.tq_encode(kc, K.view(-1, d), c["k_codes"].view(-1, kc.code_bytes), c["k_norms"].view(-1))
        tq.tq_encode(vc, V.view(-1, d), c["v_codes"].view(-1, vc.code_bytes), c["v_norms"].view(-1))
        caches.append(c)
    del K, V
    q = synth.decode_queries(B, Hq, d, device="cuda")
    ctx_len = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    out = torch.empty(B, Hq, d, device="cuda")
    ws = tq.workspace(tq.tq_attn_workspace_bytes(kc, vc, B, Hq, Hkv, ctx))
    scale = 1.0 / math.sqrt(d)
    def args_of(i):
        c = caches[i % replicas]
        return (kc, vc, q, ctx_len, c["k_codes"], c["k_norms"], c["v_codes"], c["v_norms"], scale, out, ws)

    ms, scan_ms = timed_loop(lambda i, ev: attn_step(tq, args_of(i), ev), steps, warmup, torch, probe=True)

    # the same step with a residual window of 128 exact fp16 tokens per
    # sequence (the pages' rw = 128) joining the softmax: tq_attn_decode_rw
    rw = 128
    wins = [synth.kv_block(Hkv * B, rw, d, 9000 + r, device="cuda", dtype=torch.float16) for r in range(replicas)]
    wins = [(k.view(B, Hkv, rw, d).contiguous(), v.view(B, Hkv, rw, d).contiguous()) for k, v in wins]
    win_len = torch.full((B,), rw, dtype=torch.int32, device="cuda")

    def step_rw(i, ev=None):
        c, (kw, vw) = caches[i % replicas], wins[i % replicas]
        tq.tq_attn_decode_rw(kc, vc, q, ctx_len, c["k_codes"], c["k_norms"], c["v_codes"], c["v_norms"],
                             kw, vw, win_len, scale, out, ws)

    ms_rw = timed_loop(step_rw, steps, max(warmup // 4, 1), torch)
    win_bytes = 2 * B * Hkv * rw * d * 2

    # the decode-step append: the new token's K and V of every (sequence, kv
    # head) encoded into the packed cache at ctx_len[b] (tq_append), alone and
    # followed by the attention call
    pos = torch.full((B,), ctx - 1, dtype=torch.int32, device="cuda")
    k_new, v_new = synth.kv_block(B * Hkv, 1, d, 9100, device="cuda", dtype=torch.float16)
    k_new, v_new = k_new.view(B, Hkv, d).contiguous(), v_new.view(B, Hkv, d).contiguous()

    def append(i, ev=None):
        c = caches[i % replicas]
        tq.tq_append(kc, vc, k_new, v_new, pos, c["k_codes"], c["k_norms"], c["v_codes"], c["v_norms"])

    def append_attend(i, ev=None):
        append(i)
        tq.tq_attn_decode(*args_of(i))

    ms_append = timed_loop(append, steps, max(warmup // 4, 1), torch)
    ms_append_attend = timed_loop(append_attend, steps, max(warmup // 4, 1), torch)

    # multi-query decode (speculative verification of 3 draft tokens + 1): 4
    # causal query columns per sequence in one tq_attn_decode_mq call
    C = 4
    q_mq = synth.normal((B, C, Hq, d), seed=synth.SEED_DECODE_Q + 1, dtype=torch.float16, device="cuda")
    out_mq = torch.empty(B, C, Hq, d, device="cuda")
    ws_mq = tq.workspace(tq.tq_workspace_bytes(tq.TQ_OP_ATTN_DECODE_MQ, kc, vc, B, Hq, Hkv, ctx, n_q=C))

    def mq(i, ev=None):
        c = caches[i % replicas]
        tq.tq_attn_decode_mq(kc, vc, q_mq, ctx_len, c["k_codes"], c["k_norms"], c["v_codes"], c["v_norms"], scale,
                             out_mq, ws_mq)

    ms_mq = timed_loop(mq, steps, max(warmup // 4, 1), torch)

    # the softmax-side switches on the same step (tq_attn_decode_ex): sparse V
    # at the pages' 1e-6, and dynamic sharpening (SQNR_eff 11.6)
    q1 = q.view(B, 1, Hq, d)
    out1 = out.view(B, 1, Hq, d)
    sparse_opts = tq.tq_attn_opts(tq.TQ_SCORE_PLAIN, 0.0, 0, 1e-6)
    sharp_opts = tq.tq_attn_opts(tq.TQ_SCORE_SHARPEN, 11.6, 0, 0.0)

    def step_ex(opts):
        def f(i, ev=None):
            c = caches[i % replicas]
            tq.tq_attn_decode_ex(kc, vc, q1, ctx_len, c["k_codes"], c["k_norms"], c["v_codes"], c["v_norms"], scale,
                                 out1, ws, opts)
        return f

    ms_sparse = timed_loop(step_ex(sparse_opts), steps, max(warmup // 4, 1), torch)
    ms_sharp = timed_loop(step_ex(sharp_opts), steps, max(warmup // 4, 1), torch)

    pwr = None
    if power:
        import shutil

        if shutil.which("amd-smi") is None:
            pwr = {"error": "amd-smi not found"}
        else:
            # idle board, the scan alone back to back over the rotating
            # caches, and a read-only stream of 1 GiB for comparison
            src = torch.ones((1 << 30) // 4, dtype=torch.int32, device="cuda")
            sink = torch.zeros(1, dtype=torch.int32, device="cuda")
            pwr = {
                "method": "amd-smi metric -p -c -g 0 every 0.25 s (SOCKET_POWER, mean of GFX_0..7 CLK); "
                          "first third of each run's samples dropped",
                "idle": power_probe(None, 3.0, torch),
                "scan": power_probe(lambda i: tq.tq_attn_scan(*args_of(i)), 6.0, torch),
                "stream_read_1gib": power_probe(lambda i: tq.tq_stream_read(src, sink), 6.0, torch),
            }
            del src
    token_heads = B * Hkv * ctx
    per_token_head = (kc.code_bytes + 2) + (vc.code_bytes + 2)  # 100 B
    cache_bytes = token_heads * per_token_head
    step_bytes = cache_bytes + q.numel() * 2 + out.numel() * 4
    return {
        "ms_per_step": ms,
        "gbs": step_bytes / (ms * 1e-3) / 1e9,
        "scan_ms": scan_ms,
        "scan_gbs": cache_bytes / (scan_ms * 1e-3) / 1e9,
        "cache_bytes": cache_bytes,
        "step_bytes": step_bytes,
        "bytes_per_token_head": per_token_head,
        "token_heads": token_heads,
        "replicas": replicas,
        "fma_per_token_head": 2 * g * d,
        "window": {
            "workload": "the same step plus a residual window of 128 exact fp16 tokens per sequence (tq_attn_decode_rw)",
            "win_tokens": rw,
            "ms_per_step": ms_rw,
            "gbs": (cache_bytes + win_bytes + q.numel() * 2 + out.numel() * 4) / (ms_rw * 1e-3) / 1e9,
            "window_bytes": win_bytes,
            "extra_ms_vs_packed_only": ms_rw - ms,
        },
        "multi_query": {
            "workload": "4 causal query columns per sequence (speculative verification of 3 draft tokens + 1) in one "
                        "tq_attn_decode_mq call over the same caches",
            "columns": C,
            "ms_per_call": ms_mq,
            "ms_per_column": ms_mq / C,
            "single_column_ms_per_step": ms,
            "gbs_cache_bytes": cache_bytes / (ms_mq * 1e-3) / 1e9,
        },
        "switches": {
            "workload": "the same step through tq_attn_decode_ex with one softmax-side switch on",
            "sparse_v_1e-6_ms_per_step": ms_sparse,
            "sharpen_sqnr_11.6_ms_per_step": ms_sharp,
            "plain_ms_per_step": ms,
        },
        "append": {
            "workload": "one new token per (sequence, kv head) appended to the K4 and V2 caches (one tq_append call)",
            "vectors": 2 * B * Hkv,
            "ms_per_append": ms_append,
            "ms_per_append_and_attend": ms_append_attend,
        },
        **({"power": pwr} if pwr is not None else {}),
    }, (kc, vc, caches[0], q)


# ------------------------------------------------------------------ encode ----
def encode_leg(tq, torch, synth, steps, warmup):
    H, T, d = 4, 8192, 128
    kc, vc = tq.tq_codebook(4, d, 11), tq.tq_codebook(2, d, 11)
    n = H * T
    layers = 64  # 64 x 16 MiB = 1 GiB of fp16 input
    pool_k = torch.empty(layers, n, d, dtype=torch.float16, device="cuda")
    pool_v = torch.empty(layers, n, d, dtype=torch.float16, device="cuda")
    for li in range(layers):
        k, v = synth.kv_block(H, T, d, synth.SEED_ENCODE + li, device="cuda", dtype=torch.float16)
        pool_k[li] = k.view(n, d)
        pool_v[li] = v.view(n, d)
    out_k = torch.empty(layers, n, kc.code_bytes, dtype=torch.uint8, device="cuda")
    out_v = torch.empty(layers, n, vc.code_bytes, dtype=torch.uint8, device="cuda")
    nk = torch.empty(layers, n, dtype=torch.float16, device="cuda")
    nv = torch.empty(layers, n, dtype=torch.float16, device="cuda")

    # per-layer views made once, so the timed loops call the library only
    lk, lv = [pool_k[li] for li in range(layers)], [pool_v[li] for li in range(layers)]
    lok, lov = [out_k[li] for li in range(layers)], [out_v[li] for li in range(layers)]
    lnk, lnv = [nk[li] for li in range(layers)], [nv[li] for li in range(layers)]

    def step(i, ev=None):
        li = i % layers
        tq.tq_encode(kc, lk[li], lok[li], lnk[li])
        tq.tq_encode(vc, lv[li], lov[li], lnv[li])

    ms = timed_loop(step, max(steps, 512), warmup, torch)

    def step_kv(i, ev=None):  # the same K and V through tq_encode_kv (one launch)
        li = i % layers
        tq.tq_encode_kv(kc, vc, lk[li], lv[li], lok[li], lnk[li], lov[li], lnv[li])

    ms_kv = timed_loop(step_kv, max(steps, 512), max(warmup // 4, 1), torch)

    # the same steps captured in a HIP graph (one replay = all 64 layers), the
    # way a serving loop issues them without a host call per launch
    def graph_ms(fn, replays=8):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for li in range(layers):
                fn(li)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for li in range(layers):
                fn(li)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(replays):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / (replays * layers)

    ms_graph = graph_ms(step)
    ms_kv_graph = graph_ms(step_kv)

    # single-call latency (one K+V layer), median of 20
    lat = []
    for i in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step(i)
        b.record()
        torch.cuda.synchronize()
        lat.append(a.elapsed_time(b))
    lat.sort()

    # one large launch: 2^19 keys (fp16, 4-bit) per tq_encode call over 4
    # rotating inputs (512 MiB), where the per-launch cost no longer hides the
    # kernel's own rate
    big_n = 1 << 19
    del pool_k, pool_v
    torch.cuda.empty_cache()
    big = [synth.kv_block(4, big_n // 4, d, synth.SEED_ENCODE + 100 + r, device="cuda", dtype=torch.float16)[0]
           .reshape(big_n, d) for r in range(4)]
    big_codes = torch.empty(big_n, kc.code_bytes, dtype=torch.uint8, device="cuda")
    big_norms = torch.empty(big_n, dtype=torch.float16, device="cuda")

    def step_big(i, ev=None):
        tq.tq_encode(kc, big[i % 4], big_codes, big_norms)

    ms_big = timed_loop(step_big, max(steps // 4, 20), max(warmup // 20, 5), torch)
    big_bytes = big_n * (d * 2 + kc.code_bytes + 2)
    del big
    vecs = 2 * n
    bytes_step = vecs * d * 2 + n * (kc.code_bytes + 2) + n * (vc.code_bytes + 2)
    return {
        "workload": "4 kv heads x 8192 tokens x d=128 fp16, K 4-bit + V 2-bit per step, 1 GiB rotating input pool",
        "mvectors_per_s": vecs / (ms * 1e-3) / 1e6,
        "ms_per_step": ms,
        "gbs": bytes_step / (ms * 1e-3) / 1e9,
        "bytes_per_step": bytes_step,
        "latency_ms_median": lat[len(lat) // 2],
        "steps": max(steps, 512),
        "encode_kv": {
            "call": "tq_encode_kv (K and V in one launch), same inputs and outputs",
            "mvectors_per_s": vecs / (ms_kv * 1e-3) / 1e6,
            "ms_per_step": ms_kv,
            "gbs": bytes_step / (ms_kv * 1e-3) / 1e9,
        },
        "graph": {
            "call": "the same steps captured in one HIP graph per pass over the 64 layers (no host call per launch)",
            "two_calls_mvectors_per_s": vecs / (ms_graph * 1e-3) / 1e6,
            "two_calls_ms_per_step": ms_graph,
            "encode_kv_mvectors_per_s": vecs / (ms_kv_graph * 1e-3) / 1e6,
            "encode_kv_ms_per_step": ms_kv_graph,
            "encode_kv_gbs": bytes_step / (ms_kv_graph * 1e-3) / 1e9,
        },
        "large_launch": {
            "call": "tq_encode of 2^19 fp16 keys (4-bit) per launch, 4 rotating inputs",
            "mvectors_per_s": big_n / (ms_big * 1e-3) / 1e6,
            "ms_per_launch": ms_big,
            "gbs": big_bytes / (ms_big * 1e-3) / 1e9,
            "bytes_per_launch": big_bytes,
        },
    }


# -------------------------------------------------------------------- long ----
def long_leg(tq, torch, synth, steps, warmup):
    Hkv, g, d, chunk, n_chunks = 8, 8, 128, 4096, 256
    cap = chunk * n_chunks
    kc, vc = tq.tq_codebook(3, d, 77), tq.tq_codebook(3, d, 77)
    c = {
        "k_codes": torch.empty(1, Hkv, cap, kc.code_bytes, dtype=torch.uint8, device="cuda"),
        "k_norms": torch.empty(1, Hkv, cap, dtype=torch.float16, device="cuda"),
        "v_codes": torch.empty(1, Hkv, cap, vc.code_bytes, dtype=torch.uint8, device="cuda"),
        "v_norms": torch.empty(1, Hkv, cap, dtype=torch.float16, device="cuda"),
    }
    # the 256 chunks are made first (4 GiB of bf16 K and V), then prefilled
    # back to back, as a prefill loop issues them
    chunks = [synth.long_chunk(ci, kv_heads=Hkv, tokens=chunk, d=d, device="cuda") for ci in range(n_chunks)]
    planes = (c["k_codes"][0], c["k_norms"][0], c["v_codes"][0], c["v_norms"][0])
    tq.tq_prefill(kc, vc, *chunks[0], 0, *planes)  # untimed first call (code load, launch plan)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for ci, (k, v) in enumerate(chunks):
        tq.tq_prefill(kc, vc, k, v, ci * chunk, *planes)
    b.record()
    torch.cuda.synchronize()
    enc_ms = a.elapsed_time(b)
    del chunks
    q = synth.long_queries(Hkv * g, d, device="cuda")[None].contiguous()
    ctx_len = torch.full((1,), cap, dtype=torch.int32, device="cuda")
    out = torch.empty(1, Hkv * g, d, device="cuda")
    ws = tq.workspace(tq.tq_attn_workspace_bytes(kc, vc, 1, Hkv * g, Hkv, cap))
    scale = 1.0 / math.sqrt(d)
    def args_of(i):
        return (kc, vc, q, ctx_len, c["k_codes"], c["k_norms"], c["v_codes"], c["v_norms"], scale, out, ws)

    ms, scan_ms = timed_loop(lambda i, ev: attn_step(tq, args_of(i), ev), steps, warmup, torch, probe=True)
    cache_bytes = Hkv * cap * ((kc.code_bytes + 2) + (vc.code_bytes + 2))
    return {
        "workload": "1 sequence, 8 kv heads x 2^20 tokens, d=128, K3/V3, 64 bf16 query heads (8:1)",
        "ms_per_step": ms,
        "gbs": cache_bytes / (ms * 1e-3) / 1e9,
        "scan_ms": scan_ms,
        "scan_gbs": cache_bytes / (scan_ms * 1e-3) / 1e9,
        "pct_hbm_peak": 100.0 * cache_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "cache_bytes": cache_bytes,
        "prefill_encode_ms": enc_ms,
        "prefill_encode_mvectors_per_s": 2 * Hkv * cap / (enc_ms * 1e-3) / 1e6,
    }


# ---------------------------------------------------------------- variants ----
def variants_leg(tq, torch, synth, steps, warmup):
    """Decode over the caches of the rotation, norm and head-shape variants,
    packed bytes per second with 2 cache replicas (beyond the 256 MB Infinity
    Cache):
      * head_dim 64 with the double transform S1 -> WHT -> S2 -> WHT, K4/V3
        (the head_dim-64 recommendation of [P1] v1.5.3), 8:1 GQA on the scan;
      * head_dim 512 with one norm per 256-half, K3/V3, 4:1 GQA, on the
        matrix-core wide kernel;
      * head_dim 256 with one norm per 128-half, K3/V3, 7:1 GQA, on the
        vector-ALU wide kernel;
      * head_dim 256 with one norm, K4/V3, 7:1 GQA, on the scan (4-wave blocks);
      * head_dim 128, K4/V2, 16:1 GQA, on the scan's 16-row blocks;
      * head_dim 128, K3 with Gaussian QJL signs (m = 128) / V3, 7:1 GQA."""
    out = {}
    cases = (
        ("double_wht_d64", dict(B=16, Hkv=8, g=8, ctx=32768, d=64, kb=4, vb=3, rot=tq.TQ_ROT_DOUBLE, nb=1),
         "decode, batch 16, 64 query heads / 8 kv heads, d=64, context 32768, K4/V3, double transform"),
        ("block_norm_d512", dict(B=4, Hkv=4, g=4, ctx=32768, d=512, kb=3, vb=3, rot=tq.TQ_ROT_WHT, nb=2),
         "decode, batch 4, 16 query heads / 4 kv heads, d=512, context 32768, K3/V3, two norm blocks"),
        ("block_norm_d256", dict(B=16, Hkv=4, g=7, ctx=16384, d=256, kb=3, vb=3, rot=tq.TQ_ROT_WHT, nb=2),
         "decode, batch 16, 28 query heads / 4 kv heads, d=256, context 16384, K3/V3, two norm blocks"),
        ("d256", dict(B=16, Hkv=4, g=7, ctx=16384, d=256, kb=4, vb=3, rot=tq.TQ_ROT_WHT, nb=1),
         "decode, batch 16, 28 query heads / 4 kv heads, d=256, context 16384, K4/V3"),
        ("gqa16_d128", dict(B=16, Hkv=4, g=16, ctx=32768, d=128, kb=4, vb=2, rot=tq.TQ_ROT_WHT, nb=1),
         "decode, batch 16, 64 query heads / 4 kv heads (16:1), d=128, context 32768, K4/V2"),
        ("qjl_d128", dict(B=16, Hkv=4, g=7, ctx=32768, d=128, kb=3, vb=3, rot=tq.TQ_ROT_WHT, nb=1, m=128),
         "decode, batch 16, 28 query heads / 4 kv heads, d=128, context 32768, K3 + QJL signs (m=128) / V3"),
    )
    for name, c, desc in cases:
        B, Hkv, g, ctx, d = c["B"], c["Hkv"], c["g"], c["ctx"], c["d"]
        m = c.get("m", 0)
        S = synth.qjl_projection(m, d, seed=8).cuda() if m else None
        kc = tq.tq_codebook_opts(c["kb"], d, 5, tq.TQ_RES_QJL if m else tq.TQ_RES_NONE, m, c["rot"], c["nb"])
        vc = tq.tq_codebook_opts(c["vb"], d, 5, tq.TQ_RES_NONE, 0, c["rot"], c["nb"])
        nt = (c["nb"],) if c["nb"] > 1 else ()
        caches = []
        for r in range(2):
            cc = {"k_codes": torch.empty(B, Hkv, ctx, kc.code_bytes, dtype=torch.uint8, device="cuda"),
                  "k_norms": torch.empty((B, Hkv, ctx) + nt, dtype=torch.float16, device="cuda"),
                  "v_codes": torch.empty(B, Hkv, ctx, vc.code_bytes, dtype=torch.uint8, device="cuda"),
                  "v_norms": torch.empty((B, Hkv, ctx) + nt, dtype=torch.float16, device="cuda")}
            if m:
                cc["k_qjl"] = torch.empty(B, Hkv, ctx, m // 8, dtype=torch.uint8, device="cuda")
                cc["k_gamma"] = torch.empty(B, Hkv, ctx, dtype=torch.float16, device="cuda")
            for b in range(B):
                k, v = synth.kv_block(Hkv, ctx, d, 7000 + 100 * r + b, device="cuda", dtype=torch.float16)
                tq.tq_encode_kv(kc, vc, k.view(-1, d), v.view(-1, d), cc["k_codes"][b].view(-1, kc.code_bytes),
                                cc["k_norms"][b].reshape(-1), cc["v_codes"][b].view(-1, vc.code_bytes),
                                cc["v_norms"][b].reshape(-1), S,
                                cc["k_qjl"][b].view(-1, m // 8) if m else None,
                                cc["k_gamma"][b].reshape(-1) if m else None)
            caches.append(cc)
        q = synth.normal((B, Hkv * g, d), seed=7500, dtype=torch.float16, device="cuda")
        ctx_len = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
        o_ = torch.empty(B, Hkv * g, d, device="cuda")
        ws = tq.workspace(tq.tq_attn_workspace_bytes(kc, vc, B, Hkv * g, Hkv, ctx))
        scale = 1.0 / math.sqrt(d)

        def step(i, ev=None, caches=caches, kc=kc, vc=vc, q=q, ctx_len=ctx_len, o_=o_, ws=ws, scale=scale, S=S):
            cc = caches[i % 2]
            tq.tq_attn_decode(kc, vc, q, ctx_len, cc["k_codes"], cc["k_norms"], cc["v_codes"], cc["v_norms"],
                              scale, o_, ws, cc.get("k_qjl"), cc.get("k_gamma"), S)

        ms = timed_loop(step, steps, max(warmup // 4, 1), torch)
        per = (kc.code_bytes + 2 * c["nb"]) + (vc.code_bytes + 2 * c["nb"]) + (m // 8 + 2 if m else 0)
        cache_bytes = B * Hkv * ctx * per
        out[name] = {"workload": desc, "ms_per_step": ms, "bytes_per_token_head": per, "cache_bytes": cache_bytes,
                     "gbs": cache_bytes / (ms * 1e-3) / 1e9,
                     "pct_hbm_peak": 100.0 * cache_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del caches
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ search ----
def search_leg(tq, torch, synth, steps, warmup):
    n_db, n_q, d, m, k = 1 << 20, 1024, 256, 256, 10
    db, q, S = synth.search_inputs(n_db, n_q, d, m, device="cuda")
    codec = tq.tq_codebook(3, d, 99, m)
    codes = torch.empty(n_db, codec.code_bytes, dtype=torch.uint8, device="cuda")
    norms = torch.empty(n_db, dtype=torch.float16, device="cuda")
    bits = torch.empty(n_db, m // 8, dtype=torch.uint8, device="cuda")
    gamma = torch.empty(n_db, dtype=torch.float16, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tq.tq_encode(codec, db, codes, norms, S, bits, gamma)  # first call untimed (code object load)
    a.record()
    for _ in range(3):
        tq.tq_encode(codec, db, codes, norms, S, bits, gamma)
    b.record()
    torch.cuda.synchronize()
    enc_ms = a.elapsed_time(b) / 3
    del db
    ws = tq.workspace(tq.tq_search_workspace_bytes(codec, n_q, n_db, k))
    scores = torch.empty(n_q, k, device="cuda")
    ids = torch.empty(n_q, k, dtype=torch.int64, device="cuda")

    def step(i, ev=None):
        tq.tq_ip_search(codec, q, codes, norms, bits, gamma, S, k, scores, ids, ws)

    st = max(2, min(steps, 5))
    ms = timed_loop(step, st, min(warmup, 2), torch)
    flops = 2.0 * n_q * n_db * (d + m)
    # matrix-core work actually issued: per 16 rows x 8 queries, d/16 + m/32
    # v_mfma_f32_16x16x32_f16 (2*16*16*32 flops each; the hi/lo operand fold)
    mfma_flops = n_q * n_db / 128.0 * (d // 16 + m // 32) * 2 * 16 * 16 * 32
    db_bytes = n_db * (codec.code_bytes + 2 + m // 8 + 2)
    return {
        "workload": "2^20 x 256 unit vectors, 3-bit + QJL m=256, 1024 unit queries, exact top-10",
        "ms_per_call": ms,
        "queries_per_s": n_q / (ms * 1e-3),
        "tflops": flops / (ms * 1e-3) / 1e12,
        "mfma_tflops": mfma_flops / (ms * 1e-3) / 1e12,
        "pct_fp16_mfma_peak": 100.0 * mfma_flops / (ms * 1e-3) / 1e12 / FP16_MFMA_PEAK_TFLOPS,
        "db_bytes": db_bytes,
        "db_encode_ms": enc_ms,
        "db_encode_mvectors_per_s": n_db / (enc_ms * 1e-3) / 1e6,
        "steps": st,
    }


# ----------------------------------------------------------------- quality ----
def quality_leg(tq, torch, synth):
    """Context, not parity: the tiny workload (1 kv head, d=128, 512 keys and
    values, 8 queries, 3-bit codecs) through the GPU path against exact
    uncompressed attention computed in float64 on the host -- the analogue of
    the pages' attention-score similarity and top-1 agreement figures.  MSE-only
    keys and keys with QJL (m=128): output cosine of tq_attn_decode, key-score
    cosine of q.K_hat (tq_decode), and top-1 agreement of the key scores
    (tq_ip_search with k=1, which ranks by the QJL-corrected estimate)."""
    k, v, q, S = synth.tiny()
    n, d = k.shape
    scale = 1.0 / math.sqrt(d)
    k64, v64, q64 = (t.double() for t in (k, v, q))
    s_exact = (q64 @ k64.T) * scale
    o_exact = torch.softmax(s_exact, dim=1) @ v64
    top_exact = s_exact.argmax(dim=1)
    kd, vd, qd, Sd = k.cuda(), v.cuda(), q.cuda(), S.cuda()
    vc = tq.tq_codebook(3, d, 0)
    v_codes = torch.empty(n, vc.code_bytes, dtype=torch.uint8, device="cuda")
    v_norms = torch.empty(n, dtype=torch.float16, device="cuda")
    tq.tq_encode(vc, vd, v_codes, v_norms)

    def cos_rows(a, b):
        return float((torch.nn.functional.cosine_similarity(a, b, dim=1)).mean())

    out = {"workload": "tiny: 1 kv head, d=128, 512 keys/values and 8 queries fp32 N(0,1), 3-bit K and V"}
    for name, m in (("mse", 0), ("qjl", 128)):
        kc = tq.tq_codebook(3, d, 0, m)
        k_codes = torch.empty(n, kc.code_bytes, dtype=torch.uint8, device="cuda")
        k_norms = torch.empty(n, dtype=torch.float16, device="cuda")
        bits = torch.empty(n, max(m // 8, 1), dtype=torch.uint8, device="cuda") if m else None
        gamma = torch.empty(n, dtype=torch.float16, device="cuda") if m else None
        tq.tq_encode(kc, kd, k_codes, k_norms, Sd if m else None, bits, gamma)
        o_gpu = torch.empty(1, q.shape[0], d, device="cuda")
        ws = tq.workspace(tq.tq_attn_workspace_bytes(kc, vc, 1, q.shape[0], 1, n))
        ctx = torch.tensor([n], dtype=torch.int32, device="cuda")
        tq.tq_attn_decode(kc, vc, qd[None].contiguous(), ctx, k_codes[None, None].contiguous(),
                          k_norms[None, None].contiguous(), v_codes[None, None].contiguous(),
                          v_norms[None, None].contiguous(), scale, o_gpu, ws,
                          bits[None, None].contiguous() if m else None, gamma[None, None].contiguous() if m else None,
                          Sd if m else None)
        sws = tq.workspace(tq.tq_search_workspace_bytes(kc, q.shape[0], n, 1))
        top_s = torch.empty(q.shape[0], 1, device="cuda")
        top_i = torch.empty(q.shape[0], 1, dtype=torch.int64, device="cuda")
        tq.tq_ip_search(kc, qd, k_codes, k_norms, bits, gamma, Sd if m else None, 1, top_s, top_i, sws)
        torch.cuda.synchronize()
        entry = {
            "output_cosine": cos_rows(o_gpu[0].double().cpu(), o_exact),
            "top1_agreement": float((top_i[:, 0].cpu() == top_exact).double().mean()),
        }
        if m == 0:
            k_hat = torch.empty(n, d, device="cuda")
            tq.tq_decode(kc, k_codes, k_norms, k_hat)
            torch.cuda.synchronize()
            entry["score_cosine"] = cos_rows((q64 @ k_hat.double().cpu().T) * scale, s_exact)
        out[name] = entry
    return out


# -------------------------------------------------------------- CPU oracle ----
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(torch, synth, target_s):
    """The oracle, untouched, on bounded samples of the workloads, on this
    host's cores (numpy's BLAS threads; single-thread runs under a thread limit):

    * decode (the headline unit, GB/s of packed cache): 4 (batch, kv head)
      units of the decode workload, oracle-encoded, then decompress-then-attend
      for the 7 query heads of each unit, repeated until target_s elapsed;
    * encode: the whole 4 heads x 8192 tokens fp16 K4 + V2 step (65,536
      vectors), all threads and one thread;
    * tiny: the 512-key workload (3-bit K with and without QJL m=128, 3-bit V,
      8 queries), one thread;
    * search: 64 of the 1024 queries over 2^16 of the 2^20 database rows
      (3-bit + QJL m=256, d=256, top-10), extrapolated linearly in queries x rows
      to the full call and labelled so;
    * long context: one kv head x 2^15 tokens of the K3/V3 cache with its 8
      query heads, GB/s of packed cache."""
    import numpy as np
    from oracle import tq_oracle as o

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads, threadpool_limits = 1, None

    def one_thread():
        return threadpool_limits(limits=1) if threadpool_limits else _Null()

    def f64(t):
        return t.float().numpy().astype(np.float64)

    d, ctx, g = 128, 32768, 7
    # decode sample
    kc, vc = o.Codec(4, d, 42), o.Codec(2, d, 42)
    units = [(0, 0), (5, 1), (10, 2), (15, 3)]
    caches = []
    for b, kh in units:
        k, v = synth.kv_block(4, ctx, d, synth.SEED_DECODE_BASE + b, dtype=torch.float16)
        caches.append((o.encode(f64(k[kh]), kc), o.encode(f64(v[kh]), vc)))
    q = f64(synth.decode_queries(16, 28, d))
    done, t1 = 0, time.perf_counter()
    while True:
        for (b, kh), (ek, ev) in zip(units, caches):
            o.attention(q[b, kh * g:(kh + 1) * g], ek["codes"], ek["norms"], ev["codes"], ev["norms"], kc, vc,
                        1 / math.sqrt(d))
            done += 1
        if time.perf_counter() - t1 >= target_s:
            break
    att_s = time.perf_counter() - t1
    del caches

    # encode: the whole 4 x 8192 fp16 K4 + V2 step, all threads and one thread
    k, v = synth.kv_block(4, 8192, d, synth.SEED_ENCODE, dtype=torch.float16)
    k, v = f64(k).reshape(-1, d), f64(v).reshape(-1, d)
    ek4, ev2 = o.Codec(4, d, 11), o.Codec(2, d, 11)

    def enc_step():
        t = time.perf_counter()
        o.encode(k, ek4)
        o.encode(v, ev2)
        return time.perf_counter() - t

    enc_s = enc_step()
    with one_thread():
        enc_1t_s = enc_step()
    n_enc = 2 * k.shape[0]

    # tiny workload, one thread
    kt, vt, qt, St = (x.numpy().astype(np.float64) for x in synth.tiny())
    with one_thread():
        t = time.perf_counter()
        c3, cq, cv = o.Codec(3, d, 0), o.Codec(3, d, 0, 128), o.Codec(3, d, 0)
        e_k, e_kq, e_v = o.encode(kt, c3), o.encode(kt, cq, St), o.encode(vt, cv)
        o.attention(qt, e_k["codes"], e_k["norms"], e_v["codes"], e_v["norms"], c3, cv, 1 / math.sqrt(d))
        o.attention(qt, e_kq["codes"], e_kq["norms"], e_v["codes"], e_v["norms"], cq, cv, 1 / math.sqrt(d),
                    k_qjl=e_kq["qjl"], k_gamma=e_kq["gamma"], S=St)
        tiny_s = time.perf_counter() - t

    # search sample: 64 queries x 2^16 rows, extrapolated
    n_rows, n_qs = 1 << 16, 64
    db, qs, S = synth.search_inputs(1 << 20, 1024, 256, 256)
    db, qs, S = db[:n_rows].numpy().astype(np.float64), qs[:n_qs].numpy().astype(np.float64), S.numpy()
    sc = o.Codec(3, 256, 99, 256)
    t = time.perf_counter()
    es = o.encode(db, sc, S)
    s_enc = time.perf_counter() - t
    t = time.perf_counter()
    o.ip_search(qs, es["codes"], es["norms"], es["qjl"], es["gamma"], S, sc, 10)
    s_search = time.perf_counter() - t
    del db, es
    full = s_search * (1024 / n_qs) * ((1 << 20) / n_rows)

    # long-context sample: one kv head x 2^15 tokens, 8 query heads
    lt = 1 << 15
    lk, lv = synth.long_chunk(0, kv_heads=1, tokens=lt, d=d)
    lq = f64(synth.long_queries(8, d))
    l3 = o.Codec(3, d, 77)
    elk, elv = o.encode(f64(lk[0]), l3), o.encode(f64(lv[0]), l3)
    t = time.perf_counter()
    o.attention(lq, elk["codes"], elk["norms"], elv["codes"], elv["norms"], l3, l3, 1 / math.sqrt(d))
    long_s = time.perf_counter() - t

    return {
        "value": done * ctx * 100 / att_s / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": (f"{len(units)} (batch, kv head) units of the decode workload (32768 tokens, 7 query heads each), "
                   f"oracle-encoded, then decompress-then-attend repeated {done // len(units)}x in {att_s:.1f} s"),
        "encode": {
            "workload": "the whole encode step: 4 heads x 8192 tokens fp16, K 4-bit + V 2-bit (65,536 vectors)",
            "mvectors_per_s": n_enc / enc_s / 1e6,
            "mvectors_per_s_1_thread": n_enc / enc_1t_s / 1e6,
            "seconds": enc_s,
            "seconds_1_thread": enc_1t_s,
        },
        "tiny": {
            "workload": "512 keys/values d=128, 3-bit K (MSE-only and QJL m=128) and V, 8 queries: encode + attention",
            "seconds_1_thread": tiny_s,
        },
        "search": {
            "sample": f"{n_qs} of 1024 queries over {n_rows} of 2^20 rows (3-bit + QJL m=256, d=256, top-10)",
            "sample_seconds": s_search,
            "db_encode_mvectors_per_s": n_rows / s_enc / 1e6,
            "extrapolated_ms_per_call": full * 1e3,
            "extrapolated": "linearly in queries x rows to 1024 queries over 2^20 rows",
        },
        "long": {
            "sample": f"1 of 8 kv heads x {lt} of 2^20 tokens, K3/V3, its 8 query heads (bf16)",
            "gbs": lt * 100 / long_s / 1e9,
            "seconds": long_s,
        },
    }


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def read_ceiling(tq, torch, reps=30):
    """The practical read ceiling: the library's read-only streaming kernel
    (tq_stream_read, 16-byte loads, nothing written) over a 1 GiB buffer, far
    beyond the 256 MB Infinity Cache, timed with events on the launch stream
    around each launch.  The roofline peak stays the published 8 TB/s."""
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(5):
        tq.tq_stream_read(src, sink)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        tq.tq_stream_read(src, sink)
        b.record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / reps
    del src
    return {"gbs": nbytes / (ms * 1e-3) / 1e9, "ms_per_launch": ms, "bytes": nbytes,
            "kernel": "tq_stream_read: 16-byte loads over a 1 GiB buffer, read only"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus must be 1",
                          "requested_gpus": args.gpus}))
        sys.exit(2)
    import torch

    sys.path.insert(0, ROOT)
    import synth
    import kv_cache_vector_02_amd as tq

    legs = set(args.legs.split(","))
    torch.cuda.init()
    res = {}
    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 3 launches, each 256 MiB read + 256 MiB written")
    if "decode" in legs:
        log("decode leg: batch 16, 28/4 heads, 32768 tokens, K4/V2")
        res["decode"], _ = decode_leg(tq, torch, synth, args.steps, args.warmup, power=args.power)
        log(f"decode: {res['decode']['ms_per_step']:.3f} ms/step, {res['decode']['gbs']:.0f} GB/s")
    if "encode" in legs:
        log("encode leg")
        res["encode"] = encode_leg(tq, torch, synth, args.steps, args.warmup)
        log(f"encode: {res['encode']['mvectors_per_s']:.0f} Mvectors/s")
    if "long" in legs:
        log("long-context leg (2^20 tokens)")
        res["long"] = long_leg(tq, torch, synth, max(5, args.steps // 5), max(2, args.warmup // 5))
        log(f"long: {res['long']['ms_per_step']:.3f} ms/step, {res['long']['gbs']:.0f} GB/s")
    if "search" in legs:
        log("search leg (2^20 x 256, 1024 queries)")
        res["search"] = search_leg(tq, torch, synth, args.steps, args.warmup)
        log(f"search: {res['search']['ms_per_call']:.2f} ms/call, {res['search']['tflops']:.1f} TFLOP/s")
    if "variants" in legs:
        log("variants leg (d=64 double transform, block norms at d=512 and 256, d=256, 16:1 GQA, QJL keys)")
        res["variants"] = variants_leg(tq, torch, synth, args.steps, args.warmup)
        log("variants: " + ", ".join(f"{k} {v['gbs']:.0f} GB/s" for k, v in res["variants"].items()))
    if "quality" in legs:
        res["quality"] = quality_leg(tq, torch, synth)
        log(f"quality: {res['quality']}")
    if "decode" in legs and not args.calib_copy:  # counter runs keep the calibration copies the only large ones
        res["read_ceiling"] = read_ceiling(tq, torch)
        log(f"streaming-read reference: {res['read_ceiling']['gbs']:.0f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(torch, synth, args.cpu_seconds)
        log(f"cpu: {cpu['value']:.3f} GB/s on {cpu['cores']} threads")

    dec = res.get("decode")
    line = {
        "metric": METRIC,
        "value": dec["gbs"] if dec else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"] if dec else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 operands (K scores hi/lo split, fp32-accurate), f32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": "decode attention over a packed K4/V2 cache: batch 16, 28 query heads / 4 kv heads (7:1), "
                        "d=128, context 32768, fp16 queries, scale 1/sqrt(128)",
            "batch": 16, "q_heads": 28, "kv_heads": 4, "ctx": 32768, "d": 128, "k_bits": 4, "v_bits": 2,
        },
    }
    if dec:
        line["pct_hbm_peak"] = 100.0 * dec["gbs"] / HBM_PEAK_GBS
        line["roofline"] = {
            "bound": "hbm",
            "kernel": "split-K scan (tq_attn_scan)",
            "achieved": dec["scan_gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": dec["scan_gbs"] / HBM_PEAK_GBS,
            "traffic": None,
            "scan_ms": dec["scan_ms"],
            "algorithmic_bytes_per_launch": dec["cache_bytes"],
        }
        tr = stored_traffic()
        if tr:
            line["roofline"]["traffic"] = tr["bytes"]
            line["roofline"]["traffic_detail"] = tr
        line["decode"] = dec
        if "read_ceiling" in res:
            rc = res["read_ceiling"]
            line["roofline"]["read_ceiling_gbs"] = rc["gbs"]
            line["roofline"]["frac_of_read_ceiling"] = dec["scan_gbs"] / rc["gbs"]
            line["read_ceiling"] = rc
    if cpu:
        line["cpu_baseline"] = cpu
    for k in ("encode", "long", "search", "variants", "quality"):
        if k in res:
            line[k] = res[k]
    if "encode" in res:
        line["tq_encode_mvectors_per_s"] = res["encode"]["mvectors_per_s"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
