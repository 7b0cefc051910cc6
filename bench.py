#!/usr/bin/env python3
"""Throughput of the decoder's forward pass on one MI355X.

A step is one pass of the whole hot path over one synthetic request: reset the session,
prefill the 2,048-token prompt of the Qwen3-4B-shape BF16 decoder (MFMA GEMM path, paged KV
with a shuffled 32-position block table), then 64 greedy decode steps whose token ids come
from the previous step's device-resident argmax. Inputs (weights, ids, block table) are
resident in HBM before timing starts. Prints one JSON line.

value = (prompt + decode tokens) per step / wall time per step. Prefill tok/s, decode tok/s,
their fractions of the MFMA / HBM peaks, the dominant kernel's roofline (HIP events around its
launches) and the CPU oracle on a bounded sample are reported beside it.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15    # dense FP16/BF16 MFMA, MI355X
PEAK_HBM = 8.0e12           # bytes/s, MI355X HBM3E

METRIC = "prefill tok/s @2048 + decode tok/s, Qwen3-4B-shape BF16, 1 MI355X (% roofline)"
PREFIX_PROMPT = 6890        # repeated-prompt length of the prefix-reuse measurement (Kipp Roadmap, status v0.0.3)


# bytes per projection weight: BF16; Q8_0 (34-byte blocks of 32); AFFINE4_GS32 (20-byte groups of 32)
WEIGHT_BYTES = {"bf16": 2.0, "q8_0": 34 / 32, "affine4": 20 / 32}


def algorithmic(shape, prompt, decode, scheme="bf16", kv_quant="bf16"):
    """Algorithmic FLOP of the prefill and bytes per decode token (weights + KV, no scratch).
    The prefill's output is the last position's logits plus the K/V of every position, so the
    last layer needs q|k|v for every row but attention, o and the MLP for the last row only."""
    H, F, V, L, QD = shape.hidden, shape.ffn, shape.vocab, shape.n_layers, shape.q_dim
    KVD = shape.kv_dim
    P_qkv = H * QD + 2 * H * KVD
    P = P_qkv + QD * H + 3 * H * F                                     # projection weights per layer
    attn = shape.n_q_heads * 4 * 128
    flops = (2 * (L - 1) * P * prompt + attn * (L - 1) * prompt * (prompt + 1) // 2
             + 2 * P_qkv * prompt + 2 * (P - P_qkv) + attn * prompt + 2 * V * H)
    w_bytes = int(WEIGHT_BYTES[scheme] * L * P) + 2 * (V * H + (2 * L + 1) * H + 2 * L * 128) + 2 * H
    # K and V bytes per cached position: BF16, or Q8_0 (an int8 code per value, an fp16 scale per 32)
    kv_pos = 2 * L * KVD * (2 if kv_quant == "bf16" else 34 / 32)
    ctx_mean = prompt + (decode + 1) / 2.0
    dec_bytes = w_bytes + kv_pos * ctx_mean + kv_pos
    return flops, dec_bytes, w_bytes


def cpu_baseline(wl, n_prompt, n_decode):
    """The oracle on a bounded sample of the same workload: n_prompt prompt tokens then n_decode
    greedy steps of the same model, timed after weight generation (by default the whole step:
    the 2,048-token prompt and 64 decode steps)."""
    import numpy as np
    import oracle
    import synth
    from oracle import model as om
    cores = len(os.sched_getaffinity(0))
    m = oracle.OracleModel(wl.shape, wl.weight_seed, wl.scheme)
    for l in range(wl.shape.n_layers):
        m.layer(l)
    ids = synth.token_ids(wl.ids_seed, n_prompt)
    s = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(wl.shape, n_prompt + n_decode + 1),
                             kv_quant=wl.kv_quant)
    t0 = time.perf_counter()
    lg = s.prefill(ids)
    t1 = time.perf_counter()
    for _ in range(n_decode):
        lg = s.decode(om.argmax(lg))
    t2 = time.perf_counter()
    return {"value": round((n_prompt + n_decode) / (t2 - t0), 3), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "prefill_tok_s": round(n_prompt / (t1 - t0), 3), "decode_tok_s": round(n_decode / (t2 - t1), 3),
            "sample": f"{wl.shape.name} {wl.scheme} oracle (NumPy FP32 on {cores} cores): {n_prompt}-token prompt "
                      f"+ {n_decode} greedy decode steps, weight generation untimed"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_gateup_4b_hbm_traffic.json")
# sources whose code the decode gate/up matvec is built from: its PMC traffic is reported only
# while these are unchanged since the counters were taken
TRAFFIC_SOURCES = ["dense_gqa_decoder_amd/csrc/k_gemv_full.hip", "dense_gqa_decoder_amd/csrc/gqa_common.h"]


def sources_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the decode gate/up matvec from the committed PMC summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for a plain copy of
    known size), or None when the summary is missing or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != sources_digest(TRAFFIC_SOURCES):
        return None
    return t.get("traffic_bytes_per_launch")


def blas_ceiling(reps=10):
    """Context for the prefill roofline: the vendor BLAS (torch FP16 and BF16 matmul, i.e.
    hipBLASLt) on the 4B prefill projection shapes at 2,048 tokens with random operands, as a
    measured ceiling for one FP16 matrix-core pass on this part. Not part of the product path."""
    import torch
    out = {}
    g = torch.Generator(device="cuda").manual_seed(0)
    for dt in (torch.float16, torch.bfloat16):
        for nm, N, K in (("q|k|v", 6144, 2560), ("o", 2560, 4096), ("gate|up", 19456, 2560), ("down", 2560, 9728)):
            x = (torch.rand(2048, K, device="cuda", generator=g) * 6 - 3).to(dt)
            w = ((torch.rand(N, K, device="cuda", generator=g) * 2 - 1) * 0.02).to(dt).t()
            for _ in range(3):
                x @ w
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                x @ w
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            tf = 2.0 * 2048 * N * K / (us * 1e-6) / 1e12
            out[f"{str(dt).split('.')[-1]} {nm}"] = {"us": round(us, 1), "tflops": round(tf, 1),
                                                     "frac_of_2.5pf": round(tf / 2500, 4)}
    print(json.dumps({"blas_ceiling": "torch matmul (hipBLASLt), 2048 x K x N, random operands", "shapes": out}),
          flush=True)


def pmc_workload(n_decode, chained=False):
    """The benchmark's model, prompt and decode loop without torch, for rocprofv3 --pmc passes:
    device buffers come from hipMalloc through the HIP runtime the library is linked against, and
    a 256 MiB device-to-device copy of known size follows, whose FETCH_SIZE / WRITE_SIZE readings
    calibrate the byte counters. The decode steps run with the gate/up matvec's event timing on,
    as in bench.py's roofline leg (the per-layer launches unchained, so the counted kernel is the
    one the events time), or chained as in the timed steps. Prints the copy size and exits."""
    import ctypes
    import dense_gqa_decoder_amd as g
    import synth
    g.load()
    hip = ctypes.CDLL("libamdhip64.so.7")          # the runtime already loaded by the library

    class DevBuf:
        def __init__(self, nbytes):
            p = ctypes.c_void_p()
            if hip.hipMalloc(ctypes.byref(p), ctypes.c_size_t(nbytes)) != 0:
                raise RuntimeError("hipMalloc failed")
            self.p = p.value

        def data_ptr(self):
            return self.p

    class NullStream:
        cuda_stream = None

    wl = synth.WORKLOADS["4b"]
    nb = synth.blocks_for(wl.prompt + wl.decode)
    table = synth.shuffled_blocks(wl.shuffle_seed, 4 * nb)[:nb]
    m = g.Model.from_shape(wl.shape, seed=wl.weight_seed, scheme=wl.scheme, kv_pool_blocks=4 * nb,
                           max_positions=nb * 32)
    s = g.Session(m, nb * 32, block_ids=table)
    lg, am = DevBuf(wl.shape.vocab * 4), DevBuf(4)
    s.prefill(synth.token_ids(wl.ids_seed, wl.prompt), lg, am, NullStream)
    if not chained:
        m.profile("decode_gateup")
    for _ in range(n_decode):
        s.decode(am, lg, am, NullStream)
    m.profile("none")
    size = 256 << 20
    src, dst = DevBuf(size), DevBuf(size)
    if hip.hipMemset(ctypes.c_void_p(src.p), 1, ctypes.c_size_t(size)) != 0 or \
            hip.hipMemcpy(ctypes.c_void_p(dst.p), ctypes.c_void_p(src.p), ctypes.c_size_t(size), 3) != 0 or \
            hip.hipDeviceSynchronize() != 0:
        raise RuntimeError("calibration copy failed")
    s.close()
    m.close()
    print(json.dumps({"pmc_workload": wl.shape.name, "decode_steps": n_decode, "decode_chained": chained,
                      "calibration_copy_bytes": size}), flush=True)


def pmc_batch_workload(n_steps):
    """The 8B batched workload without torch, for rocprofv3 --pmc passes: 32 sessions of contexts
    L_i ~ U{512..8192} prefilled alone, then n_steps batched decode steps of all 32."""
    import ctypes
    import dense_gqa_decoder_amd as g
    import synth
    g.load()
    hip = ctypes.CDLL("libamdhip64.so.7")

    class DevBuf:
        def __init__(self, nbytes):
            p = ctypes.c_void_p()
            if hip.hipMalloc(ctypes.byref(p), ctypes.c_size_t(nbytes)) != 0 or \
                    hip.hipMemset(p, 0, ctypes.c_size_t(nbytes)) != 0:
                raise RuntimeError("hipMalloc failed")
            self.p = p.value

        def data_ptr(self):
            return self.p

    class NullStream:
        cuda_stream = None

    wl = synth.WORKLOADS["8b-batch"]
    lens = [int(x) for x in synth.context_lengths(synth.CONTEXT_SEED_8B, wl.n_seqs)]
    need = sum(synth.blocks_for(n + n_steps) for n in lens)
    m = g.Model.from_shape(wl.shape, seed=wl.weight_seed, kv_pool_blocks=need + 64, max_positions=8192 + n_steps)
    lg, am = DevBuf(wl.shape.vocab * 4), DevBuf(4)
    sess = []
    for i, n in enumerate(lens):
        se = g.Session(m, n + n_steps)
        se.prefill(synth.token_ids(wl.ids_seed, n, offset=i * 8192), lg, am, NullStream)
        sess.append(se)
    blg, bam = DevBuf(len(sess) * wl.shape.vocab * 4), DevBuf(len(sess) * 4)
    for _ in range(n_steps):
        m.eval_batch(sess, bam, blg, bam, NullStream)
    if hip.hipDeviceSynchronize() != 0:
        raise RuntimeError("batched workload failed")
    for se in sess:
        se.close()
    m.close()
    print(json.dumps({"pmc_workload": wl.shape.name + " batched", "steps": n_steps}), flush=True)


def bench_batch(args):
    """The 8B batched workload: 32 sessions of contexts L_i ~ U{512..8192} (seed 4005), each
    prefilled alone (timed once), then a step = the workload's 128 batched decode steps of all 32
    sessions, each row greedy on its own argmax (device-resident). Prints one JSON line."""
    import numpy as np
    import torch
    import dense_gqa_decoder_amd as g
    import synth
    wl = synth.WORKLOADS["8b-batch"]
    sh = wl.shape
    lens = [int(x) for x in synth.context_lengths(synth.CONTEXT_SEED_8B, wl.n_seqs)]
    total_steps = wl.decode * (args.warmup + args.steps)
    need = sum(synth.blocks_for(n + total_steps) for n in lens)
    m = g.Model.from_shape(sh, seed=wl.weight_seed, kv_pool_blocks=need + 64, max_positions=8192 + total_steps + 32)
    stream = torch.cuda.current_stream()
    lg = torch.empty(sh.vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    sess = []
    ids = [torch.from_numpy(synth.token_ids(wl.ids_seed, n, offset=i * 8192).astype("int32")).to("cuda")
           for i, n in enumerate(lens)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, n in enumerate(lens):
        se = g.Session(m, n + total_steps)
        se.prefill(ids[i], lg, am, stream)
        sess.append(se)
    torch.cuda.synchronize()
    pre_s = time.perf_counter() - t0
    B = len(sess)
    blg = torch.empty((B, sh.vocab), device="cuda")
    bam = torch.zeros(B, dtype=torch.int32, device="cuda")

    def step():
        for _ in range(wl.decode):
            m.eval_batch(sess, bam, blg, bam, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t1) * 1e3 / args.steps
    m.check_device_error(stream)
    ctx_mean = sum(lens) / B + (args.warmup + 0.5) * wl.decode
    kv_bytes = 2 * sh.n_layers * sh.kv_dim * 2 * ctx_mean * B             # K/V read per batched step
    _, _, w_bytes = algorithmic(sh, 0, 0, wl.scheme)
    step_ms = ms_step / wl.decode
    out = {
        "metric": "batched decode tok/s, Qwen3-8B-shape BF16, 32 sessions, 1 MI355X",
        "value": round(B * wl.decode / (ms_step * 1e-3), 1), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded random-init weights, uniform random ids)",
        "config": {"workload": "qwen3-8b-shape bf16: 32 sessions, contexts %d..%d (%d positions), %d batched "
                               "decode steps per step" % (min(lens), max(lens), sum(lens), wl.decode),
                   "layers": sh.n_layers, "hidden": sh.hidden, "q_heads": sh.n_q_heads, "ffn": sh.ffn,
                   "vocab": sh.vocab, "sessions": B},
        "batched_step_ms": round(step_ms, 3),
        "prefill_s": round(pre_s, 3), "prefill_tok_s": round(sum(lens) / pre_s, 1),
        "hbm": {"weight_bytes": w_bytes, "kv_bytes_per_batched_step": int(kv_bytes),
                "achieved_gbs": round((w_bytes + kv_bytes) / (step_ms * 1e-3) / 1e9, 1),
                "frac": round((w_bytes + kv_bytes) / (step_ms * 1e-3) / PEAK_HBM, 4)},
    }
    out.update(run_record(g))
    for se in sess:
        se.close()
    m.close()
    print(json.dumps(out), flush=True)


def run_record(g):
    """Build, software and hardware record of the run (Kipp Reproducing, "Benchmarks": commit,
    dirty state, binary, compiler, hardware). The commit and dirty state are the ones baked into
    the library when it was built (git is not needed where the bench runs); "library_current"
    says whether the library's sources hash equals the current tree's, i.e. whether the binary
    measured was built from the sources beside it. Unknown facts are null, never guessed."""
    import hashlib
    import platform
    import numpy as np
    import torch
    from dense_gqa_decoder_amd import build as b
    info = g.gqa_build_info()
    with open(g.lib_path, "rb") as f:
        lib_sha = hashlib.sha256(f.read()).hexdigest()
    rocm = None
    for p in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(p) as f:
                rocm = f.read().strip()
            break
        except OSError:
            pass
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        bl = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = " ".join(str(bl.get(k)) for k in ("name", "version") if bl.get(k)) or None
    except Exception:
        pass
    dev = g.gqa_device_describe(torch.cuda.current_device())
    return {
        "commit": info.get("commit"), "dirty": info.get("dirty"),
        "library": {"sha256": lib_sha, "sources_sha256": info.get("sources_sha256"),
                    "library_current": info.get("sources_sha256") == b.sources_sha256(),
                    "hipcc": info.get("hipcc"), "flags": info.get("flags"), "built_utc": info.get("built_utc")},
        "software": {"rocm": rocm, "hip_runtime": dev["runtime_version"], "hip_driver": dev["driver_version"],
                     "torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None),
                     "python": platform.python_version(), "numpy": np.__version__},
        "device": {"name": dev["name"], "arch": dev["arch"], "cu_count": dev["cu_count"],
                   "clock_mhz": dev["clock_khz"] / 1000.0, "memory_clock_mhz": dev["memory_clock_khz"] / 1000.0,
                   "memory_bus_bits": dev["memory_bus_bits"], "memory_bytes": dev["total_memory"]},
        "host": {"cpu_model": cpu, "cores_available": len(os.sched_getaffinity(0)), "blas": blas},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="4b", choices=["4b", "0.6b", "tiny", "4b-q8", "4b-a4", "4b-kvq8",
                                                         "8b-batch"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-prompt", type=int, default=2048, help="oracle baseline: prompt tokens")
    ap.add_argument("--cpu-decode", type=int, default=64, help="oracle baseline: decode steps")
    ap.add_argument("--prefill", default="split", choices=["split", "fp16"],
                    help="prefill matrix-core operands: FP16 hi+lo (near-FP32, default) or one FP16 value")
    ap.add_argument("--pmc-workload", type=int, default=0, metavar="N",
                    help="run the 4B prompt + N decode steps and a known-size copy without torch, "
                         "for rocprofv3 --pmc passes (no timing output)")
    ap.add_argument("--pmc-chained", action="store_true",
                    help="with --pmc-workload: decode chained as in the timed steps (default: unchained, as in "
                         "the roofline leg)")
    ap.add_argument("--pmc-batch", type=int, default=0, metavar="N",
                    help="run the 8B batched workload (32 sessions, N batched steps) without torch, for "
                         "rocprofv3 --pmc passes (no timing output)")
    ap.add_argument("--blas-ceiling", action="store_true",
                    help="time the vendor BLAS on the 4B prefill GEMM shapes (context for the prefill roofline) and exit")
    args = ap.parse_args()
    if args.blas_ceiling:
        blas_ceiling()
        return
    if args.pmc_workload:
        pmc_workload(args.pmc_workload, args.pmc_chained)
        return
    if args.pmc_batch:
        pmc_batch_workload(args.pmc_batch)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: the decoder is evaluated unsharded on one MI355X "
              f"(--gpus {args.gpus} is not supported).", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_gqa_decoder_amd as g
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    g.load()
    if args.workload == "8b-batch":
        bench_batch(args)
        return
    wl = synth.WORKLOADS[args.workload]
    shape = wl.shape
    nb = synth.blocks_for(wl.prompt + wl.decode)
    pool = 4 * nb
    table = synth.shuffled_blocks(wl.shuffle_seed, pool)[:nb]
    # room for the prefix-reuse measurement's pooled sessions beside the timed one
    m = g.Model.from_shape(shape, seed=wl.weight_seed, scheme=wl.scheme,
                           kv_pool_blocks=pool + synth.blocks_for(PREFIX_PROMPT) + 1,
                           max_positions=max(nb * 32, synth.blocks_for(PREFIX_PROMPT) * 32), prefill=args.prefill,
                           kv_quant=wl.kv_quant)
    s = g.Session(m, nb * 32, block_ids=table)
    # the prompt is resident in HBM before timing (eval_prefill_device reads it there)
    ids = torch.from_numpy(synth.token_ids(wl.ids_seed, wl.prompt).astype("int32")).to("cuda")
    lg = torch.empty(shape.vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(evs=None):
        s.reset()
        if evs:
            evs[0].record(stream)
        s.prefill(ids, lg, am, stream)
        if evs:
            evs[1].record(stream)
        for _ in range(wl.decode):
            s.decode(am, lg, am, stream)
        if evs:
            evs[2].record(stream)

    # A plain device copy of known size (256 MiB read + 256 MiB written), outside the timed
    # region: under rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE calibrate the HBM byte counters.
    calib_src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    m.check_device_error(stream)
    ms_step = (t1 - t0) * 1e3 / args.steps
    pre_ms = sorted(e[0].elapsed_time(e[1]) for e in events)[args.steps // 2]
    dec_ms = sorted(e[1].elapsed_time(e[2]) for e in events)[args.steps // 2]
    tokens = wl.prompt + wl.decode
    flops, dec_bytes, w_bytes = algorithmic(shape, wl.prompt, wl.decode, wl.scheme, wl.kv_quant)

    # dominant kernel (decode gate/up matvec): HIP events around each of its launches in one
    # more step identical to the timed ones, except that while the gate/up class is recorded the
    # library issues the decode's per-layer launches unchained (a chained launch starts before its
    # predecessor ends and waits, so its events would include the wait)
    kernels = {}
    for cls in ("decode_gateup", "prefill_gateup", "prefill_attn"):
        m.profile(cls)
        step()
        n, tot_ms, dropped = m.profile_read()
        m.profile("none")
        kernels[cls] = (n, tot_ms / max(n, 1))
    H, F = shape.hidden, shape.ffn
    gu_bytes = int(2 * F * H * WEIGHT_BYTES[wl.scheme]) + H * 4 + F * 4   # weights + x hi/lo + m hi/lo, one row
    gu_ms = kernels["decode_gateup"][1]
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9
    # Prefill GEMM and attention launches: layers 0..L-2 of every round of more than 32 rows
    # (shorter rounds use the matvec; the last layer runs its MLP and attention for one row and
    # is not recorded). FLOP per launch = the class's FLOP over all its launches / launches.
    R = m.info().round_tokens
    rounds = [(o, min(R, wl.prompt - o)) for o in range(0, wl.prompt, R)]
    gemm_rounds = [(o, t) for o, t in rounds if t > 32]
    n_rec = (shape.n_layers - 1) * len(gemm_rounds)
    assert kernels["prefill_gateup"][0] == n_rec, (kernels["prefill_gateup"][0], n_rec)
    pgu_flop = sum(2.0 * t * 2 * F * H for _, t in gemm_rounds) * (shape.n_layers - 1) / n_rec
    pgu_ms = kernels["prefill_gateup"][1]
    # causal attention of a round at offset o with t rows: q.K and P.V over o + i + 1 keys for row i
    attn_unit = shape.n_q_heads * 4 * shape.head_dim
    pat_flop = sum(attn_unit * (t * o + t * (t + 1) / 2) for o, t in rounds) * (shape.n_layers - 1) / \
        max(kernels["prefill_attn"][0], 1)
    pat_ms = kernels["prefill_attn"][1]
    for name, fl, ms in (("prefill gate/up", pgu_flop, pgu_ms), ("prefill attention", pat_flop, pat_ms)):
        assert fl / (ms * 1e-3) <= PEAK_BF16_FLOPS, f"{name}: rate above the MFMA peak: accounting error"

    # Multi-row evaluation of the same prompt, outside the step: every row's logits (eval_n) and
    # the prompt's next-token scores (eval_scored), median of three, HIP events on the stream;
    # then the lm_head launches (for a round of more than 32 rows one GEMM over all its rows, else
    # the matvec over groups of up to 32 rows), timed like the kernels above.
    host_ids = synth.token_ids(wl.ids_seed, wl.prompt)
    rows_lg = torch.empty((wl.prompt, shape.vocab), device="cuda")
    rows_am = torch.empty(wl.prompt, dtype=torch.int32, device="cuda")
    scores = torch.empty(wl.prompt - 1, device="cuda")
    rows_t = []
    for _ in range(3):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        s.reset()
        ev[0].record(stream)
        s.eval_n(host_ids, rows_lg, rows_am, stream)
        ev[1].record(stream)
        s.reset()
        ev[2].record(stream)
        s.eval_scored(host_ids, scores, stream)
        ev[3].record(stream)
        torch.cuda.synchronize()
        rows_t.append((ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])))
    evn_ms = sorted(t[0] for t in rows_t)[1]
    evs_ms = sorted(t[1] for t in rows_t)[1]
    m.profile("rows_lmhead")
    s.reset()
    s.eval_n(host_ids, rows_lg, rows_am, stream)
    n_lm, lm_ms, _ = m.profile_read()
    m.profile("none")
    lm_ms /= max(n_lm, 1)
    lm_gemm = min(m.info().round_tokens, wl.prompt) > 32
    lm_rows = wl.prompt // max(n_lm, 1)                    # rows per launch
    lm_bytes = shape.vocab * shape.hidden * 2 + lm_rows * shape.hidden * 4 + lm_rows * shape.vocab * 4
    lm_flop = 2.0 * lm_rows * shape.hidden * shape.vocab
    del rows_lg

    # Prefix reuse (pooled sessions): time to the first logits of a PREFIX_PROMPT-token prompt
    # in a fresh pooled session (cold), then of the same prompt in another pooled session after
    # the first ended and published its blocks (warm: only the ids after the last whole cached
    # block are evaluated). Wall clock from the call to the logits on the host side of a
    # synchronize; median over three prompts.
    cold, warm, reused = [], [], []
    for k in range(3):
        p_ids = synth.token_ids(wl.ids_seed + 100 + k, PREFIX_PROMPT)
        for bucket in (cold, warm):
            ps = g.Session(m, synth.blocks_for(PREFIX_PROMPT) * 32, pooled=True)
            torch.cuda.synchronize()
            t_a = time.perf_counter()
            ps.prefill(p_ids, lg, am, stream)
            torch.cuda.synchronize()
            bucket.append((time.perf_counter() - t_a) * 1e3)
            if bucket is warm:
                reused.append(ps.reused)
            ps.close()
    cold_ms, warm_ms = sorted(cold)[1], sorted(warm)[1]

    out = {
        "metric": METRIC if args.workload == "4b" else
        "prefill tok/s @%d + decode tok/s, %s %s%s, 1 MI355X (%% roofline)" % (
            wl.prompt, shape.name, wl.scheme, "" if wl.kv_quant == "bf16" else ", Q8_0 KV cache"),
        "value": round(tokens / (ms_step * 1e-3), 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "q8_0": "q8_0 weights (fp16 MFMA, fp32 accumulate)",
                  "affine4": "affine4 weights (fp16 MFMA, fp32 accumulate)"}[wl.scheme],
        "data": "synthetic (seeded random-init weights ~N(0,0.02), uniform random token ids)",
        "config": {"workload": f"{shape.name} {wl.scheme}: {wl.prompt}-token prefill + {wl.decode} greedy decode "
                               f"steps, paged {'BF16' if wl.kv_quant == 'bf16' else 'Q8_0'} KV (shuffled "
                               f"32-position blocks)",
                   "kv_cache": wl.kv_quant, "kv_pool_bytes": m.info().kv_pool_bytes,
                   "layers": shape.n_layers, "hidden": shape.hidden, "q_heads": shape.n_q_heads, "kv_heads": 8,
                   "ffn": shape.ffn, "vocab": shape.vocab, "prompt": wl.prompt, "decode_steps": wl.decode,
                   "round_tokens": m.info().round_tokens},
        "prefill_tok_s": round(wl.prompt / (pre_ms * 1e-3), 1),
        "decode_tok_s": round(wl.decode / (dec_ms * 1e-3), 2),
        "prefill_ms": round(pre_ms, 3),
        "decode_ms_per_token": round(dec_ms / wl.decode, 4),
        "prefill_frac_mfma_peak": round(flops / (pre_ms * 1e-3) / PEAK_BF16_FLOPS, 4),
        "decode_frac_hbm_peak": round(dec_bytes / (dec_ms / wl.decode * 1e-3) / PEAK_HBM, 4),
        "algorithmic": {"prefill_flop": flops, "decode_bytes_per_token": int(dec_bytes), "weight_bytes": w_bytes},
        "roofline": {"kernel": "gemv_full_kernel<XF_NORM, EPI_SWIGLU>: decode gate/up matvec with fused "
                               "RMSNorm prologue and SwiGLU epilogue",
                     "bound": "hbm", "achieved": round(gu_gbs, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(gu_gbs * 1e9 / PEAK_HBM, 4), "traffic": measured_traffic() if args.workload == "4b" else None,
                     "launch_us": round(gu_ms * 1e3, 2), "bytes_per_launch": gu_bytes,
                     "launches": kernels["decode_gateup"][0]},
        "prefill_roofline": {"kernel": "gemm_kernel<EPI_SWIGLU> prefill gate/up GEMM with SwiGLU",
                             "bound": "mfma", "achieved": round(pgu_flop / (pgu_ms * 1e-3) / 1e12, 1),
                             "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                             "frac": round(pgu_flop / (pgu_ms * 1e-3) / PEAK_BF16_FLOPS, 4),
                             "launch_us": round(pgu_ms * 1e3, 1), "flop_per_launch": pgu_flop,
                             "launches": kernels["prefill_gateup"][0], "rounds": [t for _, t in rounds]},
        "prefill_attn_roofline": {"kernel": "attn_prefill_kernel: causal GQA flash attention over the paged "
                                            "BF16 KV (BF16 MFMA, q and P as BF16 hi/lo)",
                                  "bound": "mfma", "achieved": round(pat_flop / (pat_ms * 1e-3) / 1e12, 1),
                                  "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                                  "frac": round(pat_flop / (pat_ms * 1e-3) / PEAK_BF16_FLOPS, 4),
                                  "launch_us": round(pat_ms * 1e3, 1), "flop_per_launch": pat_flop,
                                  "launches": kernels["prefill_attn"][0]},
        "multi_row": {"rows": wl.prompt, "eval_n_ms": round(evn_ms, 3),
                      "eval_n_tok_s": round(wl.prompt / (evn_ms * 1e-3), 1),
                      "eval_scored_ms": round(evs_ms, 3),
                      "lm_head": {"kernel": "gemm_kernel (FP16 hi/lo, padded vocab)" if lm_gemm else "gemv_rows_kernel",
                                  "bound": "mfma" if lm_gemm else "hbm", "rows_per_launch": lm_rows,
                                  "launches": n_lm, "launch_us": round(lm_ms * 1e3, 2),
                                  "achieved_tflops": round(lm_flop / (lm_ms * 1e-3) / 1e12, 1),
                                  "frac_mfma_peak": round(lm_flop / (lm_ms * 1e-3) / PEAK_BF16_FLOPS, 4),
                                  "bytes_per_launch": lm_bytes,
                                  "achieved_gbs": round(lm_bytes / (lm_ms * 1e-3) / 1e9, 1)}},
        "prefix_reuse": {"prompt": PREFIX_PROMPT, "reused_positions": reused[1], "ttft_cold_ms": round(cold_ms, 3),
                         "ttft_warm_ms": round(warm_ms, 3), "speedup": round(cold_ms / warm_ms, 1)},
    }
    out.update(run_record(g))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, n_prompt=min(args.cpu_prompt, wl.prompt), n_decode=args.cpu_decode)
        out["cpu_baseline"].update(cpu_model=out["host"]["cpu_model"], blas=out["host"]["blas"])
    s.close()
    m.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
