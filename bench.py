"""Throughput of the audio encoder tower on one MI355X.

A step is one forward of the whole tower (conv stem, positions, every block,
final LayerNorm and the projector or pool) over one batch of synthetic clips
already resident in HBM. Prints one JSON line:

  value        audio-seconds encoded per second (30 s per full clip)
  tflops       algorithmic TFLOP/s, and mfma_frac = tflops / bf16 dense peak
  roofline     the kernel with the most time, against its own roofline, with
               its average launch time from HIP events on the forward's stream
  cpu_baseline the CPU oracle (float32 NumPy, every core of the process) on a
               bounded sample of the same workload
  ceilings     the part's own copy GB/s and bf16 MFMA-loop TFLOP/s
  configs      the other workloads: batch-1 latency (eager and HIP-graph
               replay), the variable-length batch on valid work, the stacked
               projector and the chunked attention

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "encoder audio-seconds/sec (30 s chunks, bf16, 1 GPU) + % of bf16 MFMA peak"
# MI355X published peaks: dense bf16 MFMA 2.5 PFLOP/s, fp32 157.3 TFLOP/s, HBM3E 8 TB/s.
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
PEAK_CLOCK_GHZ = 2.4        # the engine clock the published peaks are quoted at
PEAK_F32_VALU_NOPK = 78.6   # fp32 (no packed math, off in this build) and fp64 vector FMA


def step_flops(g, kind: str, rows: int, proj_rows: int) -> float:
    """Algorithmic FLOPs of one launch of a GEMM-like step over `rows` valid
    positions (`proj_rows` projector input rows: positions / stack)."""
    d, f = g.d_model, g.d_ffn
    return {
        "qkv": 2.0 * rows * d * 3 * d,
        "o_proj": 2.0 * rows * d * d,
        "fc1": 2.0 * rows * d * f,
        "fc2": 2.0 * rows * f * d,
        "proj1": 2.0 * proj_rows * g.proj_in * g.proj_hidden,
        "proj2": 2.0 * proj_rows * g.proj_hidden * g.proj_out,
    }.get(kind, 0.0)


def attention_flops(g, tb) -> float:
    """QK^T and PV over the (query, key) pairs the attention rule allows."""
    import oracle  # closed-form pair count only
    return float(sum(4.0 * oracle.attended_pairs(int(t), g.attn_chunk, g.attn_chunk_mode) * g.d_model for t in tb))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, blocks: int = 0, clips: int = 2):
    """Time the oracle (as it is, in float32 with NumPy's BLAS on every core
    this process may use) on `clips` clips of the workload: the stem, `blocks`
    of the blocks (0: all of them) and the final norm (+ projector); block
    time is scaled to the full depth when fewer blocks run."""
    from oracle import encoder as E
    from threadpoolctl import threadpool_info, threadpool_limits
    g = w.geom
    blocks = g.n_layers if blocks <= 0 else min(blocks, g.n_layers)
    W = synth.make_weights(w.replace(geom=g.replace(n_layers=blocks)))
    clips = max(1, min(clips, g.batch))
    mel = synth.make_mel(w, clips=list(range(clips)))
    mask = synth.make_mask(w, clips=list(range(clips)))
    cores = len(os.sched_getaffinity(0))
    t_stem = t_blocks = t_final = 0.0
    with threadpool_limits(limits=cores, user_api="blas"):
        blas = [{k: v for k, v in d.items() if k in ("internal_api", "version", "num_threads", "architecture",
                                                    "threading_layer")}
                for d in threadpool_info() if d.get("user_api") == "blas"]
        for c in range(clips):
            m = None if mask is None else mask[c]
            t0 = time.perf_counter()
            x = E.stem(mel[c], W, np.float32)
            t1 = time.perf_counter()
            x = E.blocks(x, W, blocks, g.n_heads, m, g.ln_eps, np.float32)
            t2 = time.perf_counter()
            E.final(x, W, g.pool_step, g.ln_eps, np.float32, g.stack)
            t3 = time.perf_counter()
            t_stem += t1 - t0
            t_blocks += t2 - t1
            t_final += t3 - t2
    measured = t_stem + t_blocks + t_final
    total = t_stem + t_blocks * g.n_layers / blocks + t_final
    frames = float(synth.make_lengths(w, clips).sum())
    return {
        "value": round(frames / 100.0 / total, 4),
        "unit": "audio-s/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{clips} clip(s) of {w.name}: stem + {blocks} of {g.n_layers} blocks + final norm"
                   f"{' + projector' if g.proj_hidden else ''}, float32 NumPy"
                   f"{'' if blocks == g.n_layers else f'; block time scaled x{g.n_layers / blocks:g}'}; "
                   f"measured {measured:.1f} s"),
        "seconds_per_clip": round(total / clips, 3),
        "tflops": round(oracle_flops(w, clips) / total / 1e12, 4),
        "cpu_model": _cpu_model(),
        "blas": blas,
    }


def oracle_flops(w, clips: int) -> float:
    import oracle  # closed-form FLOP count only
    return oracle.flops(w.geom.replace(batch=clips), synth.make_lengths(w, clips))


def measured_traffic(kind: str):
    """HBM bytes per launch of `kind` from profiles/traffic.json (rocprofv3
    FETCH_SIZE and WRITE_SIZE, scaled by the plain copy kernel's reading), or
    None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    from audio_encoder_tower_amd.rocprof_summary import source_digest
    entry = data.get("kernels", {}).get(kind)
    if not entry or entry.get("source_digest") != source_digest(kind):
        return None
    return entry.get("bytes_per_launch")


def frontend_leg(batch: int, steps: int):
    """Time the GPU log-mel front end on `batch` 30 s clips (audio resident in HBM)."""
    import torch
    import audio_encoder_tower_amd as aenc
    n = 480000
    audio = torch.from_numpy(synth.make_audio(5, batch, n)).cuda()
    fe = aenc.Frontend(batch, n, 128, out_dtype="bf16")
    out = fe(audio)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fe(audio, out)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    fe.close()
    frames = batch * (n // 160)
    # algorithmic work: real and imaginary parts of bins 0..200 over 400
    # samples (fp64), then 128 filters over the 201 bins (fp32)
    dft_flops = 2.0 * frames * 402 * 400
    mel_flops = 2.0 * frames * 128 * 201
    tf = (dft_flops + mel_flops) / (ms * 1e-3) / 1e12
    return {"workload": f"{batch} clips of 30 s, 16 kHz -> [{batch}, 128, 3000] bf16", "ms_per_batch": round(ms, 4),
            "audio_s_per_s": round(batch * 30.0 / (ms * 1e-3), 1),
            "tflops": round(tf, 2), "dft_fp64_gflop": round(dft_flops / 1e9, 2),
            # fp64 and fp32 FMA on the vector ALUs at the same full rate (no packed
            # math): 256 CUs x 64 lanes x 2 FLOP x 2.4 GHz
            "roofline": {"bound": "alu", "achieved": round(tf, 2), "peak": PEAK_F32_VALU_NOPK, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_F32_VALU_NOPK, 4)}}


def ceilings_leg(reps: int = 10):
    """The part's own ceilings, measured with the library's calibration
    kernels: a 1 GiB streaming copy (read + write bytes per second) and the
    bf16 MFMA loop on register operands (no memory traffic)."""
    import torch
    import audio_encoder_tower_amd as aenc
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.random_(0, 256)
    dst = torch.empty_like(src)
    ms_copy = timed(lambda: aenc.steps.copy_stream(dst, src), reps)
    ms_plain = timed(lambda: aenc.steps.copy(dst, src), reps)
    assert torch.equal(dst, src)
    del src, dst
    # LayerNorm's traffic without its arithmetic, on the batch-16 Whisper-large rows
    rows, d = 24064, 1280
    x = torch.randn(rows, d, device="cuda")
    y = torch.empty(rows, d, device="cuda", dtype=torch.bfloat16)
    ms_rows = timed(lambda: aenc.steps.row_stream(x, y), reps)
    assert torch.equal(y, x.to(torch.bfloat16))
    del x, y
    blocks, iters = 4096, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    ticks = torch.zeros(blocks, 2, dtype=torch.int64, device="cuda")
    flops = blocks * 4.0 * iters * 4 * 32768
    ms_mfma = timed(lambda: aenc.steps.mfma_loop(out, blocks, iters, ticks), reps)
    assert bool(torch.isfinite(out).all())
    # the shader clock the loop ran at (last launch): shader-clock over 100 MHz ticks
    t = ticks.cpu().double()
    clock_ghz = float((t[:, 0] / t[:, 1]).median()) * 0.1
    tflops = flops / (ms_mfma * 1e-3) / 1e12
    return {
        "copy_gbs": round(2 * nbytes / (ms_copy * 1e-3) / 1e9, 1),
        "copy_frac_of_8tbs": round(2 * nbytes / (ms_copy * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "copy_plain_gbs": round(2 * nbytes / (ms_plain * 1e-3) / 1e9, 1),
        "copy_bytes": 2 * nbytes,
        "row_stream_gbs": round(rows * d * 6 / (ms_rows * 1e-3) / 1e9, 1),
        "row_stream": f"{rows} rows of {d} fp32 in, bf16 out: the LayerNorm's accesses without its arithmetic",
        "mfma_bf16_tflops": round(tflops, 1),
        "mfma_frac_of_peak": round(tflops / PEAK_TFLOPS["bf16"], 4),
        # the published peak assumes 2.4 GHz; the loop's own clock scales it
        "mfma_loop_clock_ghz": round(clock_ghz, 3),
        "mfma_frac_of_peak_at_loop_clock": round(tflops / (PEAK_TFLOPS["bf16"] * clock_ghz / PEAK_CLOCK_GHZ), 4),
        "mfma_loop": f"{blocks} workgroups x 4 waves x {iters} rounds x 4 chains of 32x32x16 bf16 MFMAs",
    }


# Workloads timed beside the headline: batch-1 latency (with HIP-graph replay),
# the variable-length batch on valid work only, the stacked projector and the
# chunked attention.
CONFIG_LEGS = ["whisper_large_b1", "whisper_large_varlen_b32", "whisper_large_stack4_proj_b16", "tiny_fp32_b1",
               "whisper_medium_pool2_b1", "whisper_medium_pool2_chunk1s_b16"]


def time_forwards(enc, mel, mask, out, steps: int, warmup: int, stream):
    import torch
    for _ in range(warmup):
        enc.forward(mel, mask, out, stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        enc.forward(mel, mask, out, stream)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def time_graph_replays(enc, mel, mask, out, steps: int):
    """One forward captured into a HIP graph, then `steps` replays."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        enc.forward(mel, mask, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        enc.forward(mel, mask, out)
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    del graph
    return a.elapsed_time(b) / steps


def device_weights(w, cache: dict, tdt):
    """Device copies of the workload's weights, reusing the encoder part and
    the projector part across workloads that share their seeds and shapes
    (each tensor has its own seeded stream, so the values are the same)."""
    import torch
    g = w.geom
    enc_key = ("enc", w.weight_seed, w.init, g.dtype, g.n_mel, g.d_model, g.n_layers, g.d_ffn)
    proj_key = ("proj", w.proj_seed, w.init, g.dtype, g.proj_in, g.proj_hidden, g.proj_out)
    for k in [k for k in cache if k not in (enc_key, proj_key)]:
        del cache[k]
    if enc_key not in cache:
        W = synth.make_weights(w.replace(geom=g.replace(proj_hidden=0, proj_out=0, stack=1)))
        cache[enc_key] = {k: torch.from_numpy(v).to("cuda").to(tdt) for k, v in W.items()}
    out = dict(cache[enc_key])
    if g.proj_hidden:
        if proj_key not in cache:
            # projector tensors draw from their own seed: the same values whatever the depth
            W = synth.make_weights(w.replace(geom=g.replace(n_layers=0)))
            cache[proj_key] = {k: torch.from_numpy(v).to("cuda").to(tdt) for k, v in W.items()
                               if k.startswith("proj")}
        out.update(cache[proj_key])
    return out


def configs_leg(names, steps: int, warmup: int, weights_cache: dict):
    """Each workload in `names` timed like the headline (inputs resident in
    HBM, HIP events on the forward's stream). Batch-1 workloads also report
    HIP-graph replay of the same forward."""
    import torch
    import audio_encoder_tower_amd as aenc
    import oracle  # closed-form FLOP count only
    out_rec = {}
    stream = torch.cuda.current_stream()
    for name in names:
        w = synth.get_workload(name)
        g = w.geom
        tdt = torch.bfloat16 if g.dtype == "bf16" else torch.float32
        enc = aenc.Encoder(g, device_weights(w, weights_cache, tdt))
        mel = torch.from_numpy(synth.make_mel(w)).to("cuda").to(tdt)
        mask_np = synth.make_mask(w)
        mask = None if mask_np is None else torch.from_numpy(mask_np).to("cuda")
        out = torch.empty(enc.out_shape, dtype=enc.out_dtype, device="cuda")
        n = steps if g.batch > 1 else 5 * steps
        ms = time_forwards(enc, mel, mask, out, n, warmup, stream)
        frames = synth.make_lengths(w)
        fl = oracle.flops(g, frames)
        audio_s = float(frames.sum()) / 100.0
        peak = PEAK_TFLOPS[g.dtype]
        rec = {"batch": g.batch, "dtype": g.dtype, "ms_per_forward": round(ms, 4),
               "audio_s_per_s": round(audio_s / (ms * 1e-3), 1), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
               "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / peak, 4), "flops_per_forward": fl,
               "audio_s_per_forward": audio_s}
        if w.varlen:
            rec["valid_frames"] = int(frames.sum())
            rec["padded_frames"] = int(g.batch * g.n_frames)
            rec["counted"] = "valid positions and key pairs only"
        if g.batch == 1:
            gms = time_graph_replays(enc, mel, mask, out, n)
            rec["graph_ms_per_forward"] = round(gms, 4)
            rec["graph_audio_s_per_s"] = round(audio_s / (gms * 1e-3), 1)
        enc.close()
        del mel, mask, out
        out_rec[name] = rec
        print(f"config {name}: {rec}", file=sys.stderr, flush=True)
    weights_cache.clear()
    torch.cuda.empty_cache()
    return out_rec


def cache_leg(enc, mel, mask, out, audio_s: float, steps: int):
    """The embeddings cache on the bench batch: one forward that fills it (all
    misses), then all-hit batches served by device copies."""
    import torch
    import audio_encoder_tower_amd as aenc
    g = enc.geom
    cache = aenc.EmbeddingsCache.for_encoder(enc, 2 * g.batch)
    keys = list(range(1000, 1000 + g.batch))
    stream = torch.cuda.current_stream()
    start, mid, end = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    torch.cuda.synchronize()
    start.record(stream)
    _, hits0 = enc.forward_cached(cache, keys, mel, mask, out, stream)
    mid.record(stream)
    for _ in range(steps):
        _, hits = enc.forward_cached(cache, keys, mel, mask, out, stream)
    end.record(stream)
    torch.cuda.synchronize()
    miss_ms, hit_ms = start.elapsed_time(mid), mid.elapsed_time(end) / steps
    nbytes = out.numel() * out.element_size()
    stats = cache.stats()
    cache.close()
    return {"entries": g.batch, "entry_bytes": nbytes // g.batch, "first_batch_hits": hits0, "hits_per_batch": hits,
            "miss_batch_ms": round(miss_ms, 3), "hit_batch_ms": round(hit_ms, 4),
            "hit_copy_gbs": round(2 * nbytes / (hit_ms * 1e-3) / 1e9, 1),
            "hit_audio_s_per_s": round(audio_s / (hit_ms * 1e-3), 1), "stats": stats}


def side_stream_leg(enc, mel, mask, out, audio_s: float, n_enc: int = 4, gate_forwards: int = 3, shape=None,
                    enc_stream=None, dec_stream=None):
    """The encoder on a stream of its own while a decode-like load (synth.decode_load)
    runs on another, against each alone.

    Every run starts behind a gate: `gate_forwards` encoder forwards on a third
    stream, after which an event releases the measured streams; the host
    enqueues all measured work while the gate holds, so the times are the
    GPU's and not the host's launch rate. The decode side takes as many steps
    as last about as long as the encoder's `n_enc` forwards alone.
    overlap_efficiency = (serial - concurrent) / (serial - max(alone)): 1 when
    both finish as if each had the GPU to itself, 0 when no better than
    running one after the other."""
    import torch
    from synth.decode_load import DecodeLoad, KIMI_AUDIO_LLM
    shape = shape or KIMI_AUDIO_LLM
    load = DecodeLoad(shape)
    sa = enc_stream or torch.cuda.Stream()
    sb = dec_stream or torch.cuda.Stream()
    sg = torch.cuda.Stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def dec(n):
        with torch.cuda.stream(sb):
            for _ in range(n):
                load.step()

    def gated(streams, enqueue):
        torch.cuda.synchronize()
        for _ in range(gate_forwards):
            enc.forward(mel, mask, out, sg)
        g0 = ev()
        g0.record(sg)
        for s in streams:
            s.wait_event(g0)
        t0 = time.perf_counter()
        enqueue()
        host_ms = (time.perf_counter() - t0) * 1e3
        ends = []
        for s in streams:
            e = ev()
            e.record(s)
            ends.append(e)
        torch.cuda.synchronize()
        return [g0.elapsed_time(e) for e in ends], host_ms

    dec(2)                                               # library warm-up
    enc.forward(mel, mask, out, sa)
    (t3,), _ = gated([sb], lambda: dec(3))
    t_step = t3 / 3
    (t_enc,), _ = gated([sa], lambda: [enc.forward(mel, mask, out, sa) for _ in range(n_enc)])
    n_dec = max(1, round(t_enc / t_step))
    (t_dec,), _ = gated([sb], lambda: dec(n_dec))

    def both():
        done = 0
        for i in range(n_enc):
            enc.forward(mel, mask, out, sa)
            k = round(n_dec * (i + 1) / n_enc) - done
            dec(k)
            done += k

    (ta, tb), host_ms = gated([sa, sb], both)
    t_both = max(ta, tb)
    serial, ideal = t_enc + t_dec, max(t_enc, t_dec)
    del load
    torch.cuda.synchronize()
    return {
        "load": f"decode of {shape.tokens} rows through {shape.layers} layers (hidden {shape.hidden}, kv "
                f"{shape.kv_dim}, intermediate {shape.inter}): {shape.weight_bytes() / 1e9:.2f} GB of bf16 weights "
                f"per step",
        "encoder_forwards": n_enc, "decode_steps": n_dec,
        "encoder_alone_ms": round(t_enc, 3), "decode_alone_ms": round(t_dec, 3),
        "decode_step_alone_ms": round(t_dec / n_dec, 4),
        "decode_alone_gbs": round(shape.weight_bytes() * n_dec / (t_dec * 1e-3) / 1e9, 1),
        "concurrent_ms": round(t_both, 3), "encoder_done_ms": round(ta, 3), "decode_done_ms": round(tb, 3),
        "encoder_audio_s_per_s_under_load": round(audio_s * n_enc / (ta * 1e-3), 1),
        "speedup_vs_serial": round(serial / t_both, 4),
        "overlap_efficiency": round((serial - t_both) / (serial - ideal), 4) if serial > ideal else None,
        "host_enqueue_ms": round(host_ms, 2),
        "gate_ms_alone": round(t_enc / n_enc * gate_forwards, 2),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=synth.workloads.HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-blocks", type=int, default=0, help="blocks the CPU oracle runs (0: all)")
    ap.add_argument("--no-frontend", action="store_true", help="skip timing the log-mel front end")
    ap.add_argument("--no-side-stream", action="store_true",
                    help="skip the encoder-beside-decode overlap measurement")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run the plain copy kernel over this many MiB (a reference for traffic counters)")
    ap.add_argument("--cpu-clips", type=int, default=2, help="clips the CPU oracle encodes")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other workloads (batch-1 latency, variable length, stacked, chunked)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the copy and MFMA-loop ceilings")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.exit("bench.py runs on one GPU only: the encoder's clips are independent, and this build "
                 "measures one GPU's share (see the sharding notes); use --gpus 1")

    import torch
    import audio_encoder_tower_amd as aenc

    assert torch.cuda.is_available(), "no HIP device"
    w = synth.get_workload(args.workload)
    g = w.geom
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.bfloat16 if g.dtype == "bf16" else torch.float32

    weights_cache = {}
    enc = aenc.Encoder(g, device_weights(w, weights_cache, tdt))
    mel = torch.from_numpy(synth.make_mel(w)).to(dev).to(tdt)
    mask_np = synth.make_mask(w)
    mask = None if mask_np is None else torch.from_numpy(mask_np).to(dev)
    out = torch.empty(enc.out_shape, dtype=enc.out_dtype, device=dev)
    stream = torch.cuda.current_stream()

    frames = synth.make_lengths(w)
    tb = (frames + 1) // 2
    audio_s = float(frames.sum()) / 100.0
    import oracle  # closed-form FLOP count only
    flops = oracle.flops(g, frames)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        aenc.steps.copy(dst, src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        enc.forward(mel, mask, out, stream)
    torch.cuda.synchronize()

    # ---- timed region ----
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        enc.forward(mel, mask, out, stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps

    # ---- per-kernel times: HIP events around every launch, same stream ----
    enc.profile(True)
    for _ in range(args.steps):
        enc.forward(mel, mask, out, stream)
    torch.cuda.synchronize()
    kinds = enc.profile_read()
    enc.profile(False)

    rows = int(tb.sum())
    proj_rows = int((tb // g.stack).sum())
    per_kind = {}
    for k, (ms, n) in sorted(kinds.items(), key=lambda kv: -kv[1][0]):
        avg = ms / n
        entry = {"ms_per_step": round(ms / args.steps, 4), "launches_per_step": n // args.steps,
                 "avg_launch_ms": round(avg, 5)}
        fl = step_flops(g, k, rows, proj_rows) if k != "attention" else attention_flops(g, tb)
        if fl:
            entry["tflops"] = round(fl / (avg * 1e-3) / 1e12, 1)
        if k == "layernorm":   # fp32 rows in, bf16 (or fp32) rows out
            nbytes = rows * g.d_model * (4 + (2 if g.dtype == "bf16" else 4))
            entry["gbs"] = round(nbytes / (avg * 1e-3) / 1e9, 1)
        if w.name == synth.workloads.HEADLINE:
            t = measured_traffic(k)   # counter bytes per launch, taken on this workload
            if t:
                entry["counter_bytes_per_launch"] = t
        per_kind[k] = entry
    dominant = max(kinds, key=lambda k: kinds[k][0])
    dom_ms, dom_n = kinds[dominant]
    dom_avg = dom_ms / dom_n
    dom_flops = step_flops(g, dominant, rows, proj_rows) if dominant != "attention" else attention_flops(g, tb)
    peak = PEAK_TFLOPS[g.dtype]
    roofline = {
        "kernel": dominant,
        "bound": "mfma",
        "achieved": round(dom_flops / (dom_avg * 1e-3) / 1e12, 1),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(dom_flops / (dom_avg * 1e-3) / 1e12 / peak, 4),
        "traffic": measured_traffic(dominant),
        "avg_launch_ms": round(dom_avg, 5),
        "flops_per_launch": dom_flops,
    }

    tflops = flops / (ms_step * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(audio_s / (ms_step * 1e-3), 1),
        "unit": "audio-s/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": g.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "global_batch": g.batch, "seq_len": g.n_pos, "mel_frames": g.n_frames,
                   "d_model": g.d_model, "layers": g.n_layers, "heads": g.n_heads, "ffn": g.d_ffn,
                   "pool_step": g.pool_step, "stack": g.stack,
                   "attn_chunk": [g.attn_chunk, {0: "none", 1: "causal", 2: "block"}[g.attn_chunk_mode]],
                   "projector": [g.proj_in, g.proj_hidden, g.proj_out] if g.proj_hidden else None,
                   "audio_seconds_per_step": audio_s, "parallelism": "none (1 GPU)"},
        "tflops": round(tflops, 1),
        "mfma_frac": round(tflops / peak, 4),
        "flops_per_step": flops,
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "kernels": per_kind,
    }
    print(f"headline {w.name}: {ms_step:.3f} ms per forward", file=sys.stderr, flush=True)
    if not args.no_frontend:
        result["frontend"] = frontend_leg(g.batch, args.steps)
    if not args.no_side_stream:
        result["side_stream"] = side_stream_leg(enc, mel, mask, out, audio_s)
        result["cache"] = cache_leg(enc, mel, mask, out, audio_s, args.steps)
    enc.close()
    if not args.no_ceilings:
        c = ceilings_leg()
        result["ceilings"] = c
        # the same kernels against the part's own ceilings
        roofline["frac_of_measured_ceiling"] = round(roofline["achieved"] / c["mfma_bf16_tflops"], 4)
        result["mfma_frac_of_measured_ceiling"] = round(tflops / c["mfma_bf16_tflops"], 4)
        if "layernorm" in per_kind:
            per_kind["layernorm"]["frac_of_copy_ceiling"] = round(per_kind["layernorm"]["gbs"] / c["copy_gbs"], 4)
            per_kind["layernorm"]["frac_of_row_stream"] = round(per_kind["layernorm"]["gbs"] / c["row_stream_gbs"], 4)
        print(f"ceilings: {c}", file=sys.stderr, flush=True)
    if not args.no_configs:
        result["configs"] = configs_leg([n for n in CONFIG_LEGS if n != w.name], args.steps, args.warmup,
                                        weights_cache)
    weights_cache.clear()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_blocks, args.cpu_clips)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
