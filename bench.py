"""Benchmark of KV-cache transform coding on one MI355X.

Default workload (llama31_8b): Llama-3.1-8B-shaped cache, 32 layers x {K, V},
8 kv heads x 128 = 1024 features, 8192 tokens, bf16, sink 4, window 128, 16x
budget (1 bit per value), microscale group 16; seeded synthetic KV (shared
96-dim latent per layer, per-head rotations, power-law spectrum, 4 outlier key
channels per head), calibrated on 16384 synthetic tokens per tensor by the
library on the host.

One step = kvtc_encode of every tensor followed by kvtc_decode of every
stream back to bf16 (one launch per 32 tensors per kernel), with inputs,
streams and outputs resident in HBM; kvtc_decode gets its full workspace and
so runs the two-stage schedule (stage 1 unpacks records into MFMA operands in
a staging buffer, stage 2 restores). HIP events on the launch stream time the
encode and the decode inside the timed region. value = bf16 KV bytes per
step / step time. After the timed steps the same step runs on for about
250 ms and its last 50 steps are reported as `sustained` (the GPU needs
some 100-200 ms of this load to reach its steady kernel times, so a short
timed run measures part of that ramp); then the step's decode call is timed
in a loop of its own (`decode_alone`), the same two stages with an event
between them (the per-kernel breakdown), the encode of a copy of the codec
whose slots all take the centred product (`encode_centred`: the path of
slots whose mean exceeds their spread), and kvtc_decode with only
the status words (the single-launch fused schedule) is timed on its own.
Then the online encode: layer l + 1's K and V are produced (a bf16 GEMM per
tensor standing in for the model's projections) on one stream while layer l
is encoded on another (`online_encode`).
For a paged workload (qwen25_7b_paged) the decode is the layer-by-layer
two-stream pipeline: stage 1 (unpack) of layer l+1 runs on one stream while
stage 2 (restore into the paged cache) of layer l runs on another. The
DEFLATE ratio (host zlib) is reported outside the timed region.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# device code the traffic counters in profiles/traffic.json were taken on
KERNEL_SOURCES = ("kvtc_device.h", "kvtc_encode.hip", "kvtc_decode.hip", "kvtc_internal.h")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama31_8b")
    ap.add_argument("--cpu-sample", type=int, default=16, help="most tensors in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-schedule", choices=("staged", "fused"), default="staged",
                    help="kvtc_decode's workspace in the timed step: with the staging (the "
                         "two-stage schedule) or only the status words (the fused schedule)")
    ap.add_argument("--calib-tokens", type=int, default=0, help="override (0 = workload's)")
    ap.add_argument("--distinct-requests", type=int, default=2,
                    help="distinct synthetic requests per (layer, kind); the rest are copies")
    ap.add_argument("--pipeline-buffers", type=int, default=2,
                    help="paged workloads: staging buffers of the two-stream layer pipeline")
    ap.add_argument("--core-only", action="store_true",
                    help="only the step and its per-kernel loops (no lossless stage or online "
                         "encode sections): for profiler runs whose per-kernel averages must "
                         "cover the step's launches alone")
    ap.add_argument("--save-artifact", default="", help="write the calibrated artifact here")
    ap.add_argument("--load-artifact", default="",
                    help="use this artifact (written by --save-artifact for the same workload) "
                         "instead of calibrating")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU: the path is not sharded here (--gpus must be 1)"}))
        sys.exit(2)

    import torch
    import kv_cache_transform_amd as K
    import synth

    w = synth.workload(args.workload)
    dt = K.KVTC_BF16 if w.dtype == "bf16" else K.KVTC_F32
    cores = len(os.sched_getaffinity(0))
    kp = K.params(w.n_layers, w.kv_heads, w.head_dim, w.sink, w.window, w.group, 8,
                  w.bits_per_value, dt)
    if args.load_artifact:
        with open(args.load_artifact, "rb") as f:
            codec = K.Codec.load(f.read())
    else:
        codec = K.Codec(kp)
    slots = [(l, k) for l in range(w.n_layers) for k in w.kinds]
    calib_n = args.calib_tokens or w.calib_tokens

    # --- calibration on the host (library), one worker per slot in flight
    t0 = time.time()
    workers = max(1, min(16, cores))
    per = max(1, cores // workers)

    def calib(slot):
        l, k = slot
        x = synth.storage(w, synth.gen_kv(w, l, k, synth.ROLE_CALIB, calib_n))
        codec.calibrate(l, k, x, threads=per)

    if not args.load_artifact:
        with cf.ThreadPoolExecutor(workers) as ex:
            for i, _ in enumerate(ex.map(calib, slots)):
                if (i + 1) % 16 == 0:
                    log(f"calibrated {i + 1}/{len(slots)} slots ({time.time() - t0:.1f}s)")
        if args.save_artifact:
            with open(args.save_artifact, "wb") as f:
                f.write(codec.save())
    calib_s = time.time() - t0
    infos = {s: codec.slot(*s) for s in slots}

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    n_state = codec.state_bytes()
    state = torch.empty(n_state, dtype=torch.uint8, device=dev)
    codec.upload(state, n_state, stream)

    # --- jobs: every (layer, kind, request); inputs, streams, outputs resident
    T, F = w.n_tokens, w.features
    esz = w.elem_bytes
    R = w.n_requests
    jobs = [(l, k, r) for l in range(w.n_layers) for k in w.kinds for r in range(R)]
    n_jobs = len(jobs)
    tdt = torch.int16 if dt == K.KVTC_BF16 else torch.float32
    xs = torch.empty((n_jobs, T, F), dtype=tdt, device=dev)
    n_distinct = max(1, min(R, args.distinct_requests))
    for i, (l, k, r) in enumerate(jobs):
        if r < n_distinct:
            st = synth.storage(w, synth.gen_kv(w, l, k, synth.ROLE_EVAL, T, r))
            xs[i].copy_(torch.from_numpy(st.view(np.int16) if dt == K.KVTC_BF16 else st))
        else:
            xs[i].copy_(xs[i - r + r % n_distinct])
    sizes = [codec.encoded_bytes(l, k, T) for l, k, _ in jobs]
    offs = np.cumsum([0] + [(n + 255) // 256 * 256 for n in sizes])
    sbuf = torch.zeros(int(offs[-1]), dtype=torch.uint8, device=dev)
    ws = torch.zeros(K.kvtc_workspace_bytes(n_jobs) // 4, dtype=torch.int32, device=dev)
    enc_jobs = [K.make_job(l, k, T, xs[i], sbuf.data_ptr() + int(offs[i]), sizes[i])
                for i, (l, k, _) in enumerate(jobs)]
    if w.paged:
        # Each (layer, kind) owns a pool of R * ceil(T / bs) blocks; every
        # request gets a random disjoint subset of it as its block table.
        bs = w.block_size
        per_req = (T + bs - 1) // bs
        rng = np.random.default_rng(11)
        tables = torch.empty((n_jobs, per_req), dtype=torch.int32)
        pools = {}
        for i, (l, k, r) in enumerate(jobs):
            if (l, k) not in pools:
                pools[(l, k)] = rng.permutation(R * per_req).astype(np.int32)
            tables[i] = torch.from_numpy(pools[(l, k)][r * per_req:(r + 1) * per_req])
        tables = tables.to(dev)
        out = torch.empty((len(slots), R * per_req * bs, F), dtype=torch.int16, device=dev)
        pool_of = {s: i for i, s in enumerate(slots)}
        dec_jobs = [K.make_job(l, k, T, sbuf.data_ptr() + int(offs[i]), out[pool_of[(l, k)]],
                               out[pool_of[(l, k)]].numel() * 2, tables[i], bs, R * per_req,
                               src_capacity=sizes[i])
                    for i, (l, k, _) in enumerate(jobs)]
    else:
        out = torch.empty((n_jobs, T, F), dtype=torch.int16, device=dev)
        dec_jobs = [K.make_job(l, k, T, sbuf.data_ptr() + int(offs[i]), out[i], out[i].numel() * 2,
                               src_capacity=sizes[i])
                    for i, (l, k, _) in enumerate(jobs)]
    log(f"calibration {calib_s:.1f}s; state {n_state / 2**20:.1f} MiB; "
        f"streams {offs[-1] / 2**20:.1f} MiB; {n_jobs} tensors")

    def encode():
        codec.encode(enc_jobs, ws, stream)

    pipe = Pipeline(K, codec, w, jobs, dec_jobs, dev, args.pipeline_buffers) if w.paged else None

    # kvtc_decode's full workspace (status words, sink, staging) selects the
    # two-stage schedule; the status words alone, the fused one
    n_dws = codec.decode_workspace_bytes(dec_jobs)
    n_ws0 = K.kvtc_workspace_bytes(n_jobs)
    dws = torch.zeros((n_dws + 3) // 4, dtype=torch.int32, device=dev)
    # staging for the explicit stage calls of the per-kernel breakdown
    n_stg = codec.staging_bytes(dec_jobs)
    stg = torch.empty(max(n_stg, 256), dtype=torch.uint8, device=dev)

    n_step_ws = n_dws if args.decode_schedule == "staged" else n_ws0

    def decode():
        if pipe is not None:
            pipe.run(stream)
        else:
            codec.decode(dec_jobs, K.KVTC_BF16, dws, n_step_ws, stream)

    def decode_fused():
        codec.decode(dec_jobs, K.KVTC_BF16, dws, n_ws0, stream)

    def decode_staged(mid):
        codec.decode_unpack(dec_jobs, K.KVTC_BF16, stg, n_stg, dws, stream)
        mid.record(stream)
        codec.decode_restore(dec_jobs, K.KVTC_BF16, stg, n_stg, dws, stream)

    # Plain device copy of a known size: the practical HBM ceiling and the
    # reference that scales the FETCH_SIZE / WRITE_SIZE counters.
    copy_bytes = 1 << 30
    csrc = torch.empty(copy_bytes // 2, dtype=torch.int16, device=dev)
    cdst = torch.empty_like(csrc)
    for _ in range(2):
        cdst.copy_(csrc)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        cdst.copy_(csrc)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * copy_bytes * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del csrc, cdst

    for _ in range(args.warmup):
        encode()
        decode()
    torch.cuda.synchronize()
    st = K.kvtc_read_device_status(ws, n_jobs, stream)
    if pipe is None:
        st = np.concatenate([st, K.kvtc_read_device_status(dws, n_jobs, stream)])
    if np.any(st != 0):
        raise SystemExit(f"device status errors: {st}")
    if pipe is not None:
        pipe.check()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        encode()
        e1.record(stream)
        decode()
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    enc_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
    dec_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    ms_per_step = wall * 1e3 / args.steps
    # The same step sustained for about a quarter of a second more: the GPU
    # takes some 100-200 ms of this load to settle at its steady kernel
    # times, so a short timed run measures part of that ramp. The last 50
    # steps give the sustained figures reported beside the timed ones.
    n_sus = max(60, int(250.0 / max(ms_per_step, 1e-3)))
    evu = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_sus)]
    for u0, u1, u2 in evu:
        u0.record(stream)
        encode()
        u1.record(stream)
        decode()
        u2.record(stream)
    torch.cuda.synchronize()
    sus_enc = np.array([a.elapsed_time(b) for a, b, _ in evu[-50:]])
    sus_dec = np.array([b.elapsed_time(c) for _, b, c in evu[-50:]])
    # the step's decode call alone, back to back
    eva = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for a0, a1 in eva:
        a0.record(stream)
        decode()
        a1.record(stream)
    torch.cuda.synchronize()
    alone_ms = np.array([a.elapsed_time(b) for a, b in eva])
    if pipe is None:
        # per-kernel breakdown of the decode (same calls, an event between the stages)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for d0, d1, d2 in evs:
            d0.record(stream)
            decode_staged(d1)
            d2.record(stream)
        torch.cuda.synchronize()
        prep_ms = np.array([a.elapsed_time(b) for a, b, _ in evs])
        gemm_ms = np.array([b.elapsed_time(c) for _, b, c in evs])
        evf = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for f0, f1 in evf:
            f0.record(stream)
            decode_fused()
            f1.record(stream)
        torch.cuda.synchronize()
        fused_ms = np.array([a.elapsed_time(b) for a, b in evf])
        if np.any(K.kvtc_read_device_status(dws, n_jobs, stream) != 0):
            raise SystemExit("device status errors in the fused decode")

    # The same encode with every slot on the centred product (two MFMA
    # terms per token), the path of slots whose mean exceeds their spread:
    # a copy of the codec finished with KVTC_ENCODE_CENTRED=1.
    cen_ms = None
    n_fold = sum(infos[sl].folded_mean for sl in slots)
    if dt == K.KVTC_BF16 and n_fold and not args.core_only:
        os.environ["KVTC_ENCODE_CENTRED"] = "1"
        try:
            codec_c = K.Codec.load(codec.save())
        finally:
            del os.environ["KVTC_ENCODE_CENTRED"]
        assert all(codec_c.slot(*sl).folded_mean == 0 for sl in slots)
        state_c = torch.empty(codec_c.state_bytes(), dtype=torch.uint8, device=dev)
        codec_c.upload(state_c, state_c.numel(), stream)
        evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for c0, c1 in evc:
            c0.record(stream)
            codec_c.encode(enc_jobs, ws, stream)
            c1.record(stream)
        torch.cuda.synchronize()
        if np.any(K.kvtc_read_device_status(ws, n_jobs, stream) != 0):
            raise SystemExit("device status errors in the centred encode")
        cen_ms = np.array([a.elapsed_time(b) for a, b in evc])
        del state_c

    kv_bytes = n_jobs * T * F * esz
    r_eff = {s: infos[s].r_eff for s in slots}
    n_launch = (n_jobs + 31) // 32
    stream_total = int(sum(sizes))
    tc = T - min(w.sink, T) - min(w.window, T - min(w.sink, T))
    pass_rows = T - tc
    # Algorithmic HBM bytes of one call of each kernel, per launch: what the
    # kernel must read and write at least.
    #  encode: the KV rows, the streams, the bf16 basis per tensor, and its
    #          fp32 mean (f32 input) or the mean's projection mu V' (bf16 input)
    #  fused decode: the streams, the KV rows out, fp16 basis + mean
    #  decode stage 1: the streams, the staging it writes, passthrough rows out
    #  decode stage 2: the staging, the compressed rows out, fp16 basis + mean
    staging = n_stg
    r_enc = {s: (r + 31) // 32 * 32 for s, r in r_eff.items()}
    enc_alg = kv_bytes + stream_total + sum(r_enc[(l, k)] * F * 2 + (F * 4 if esz == 4 else r_enc[(l, k)] * 4)
                                            for l, k, _ in jobs)
    prep_alg = stream_total + staging + n_jobs * pass_rows * F * esz
    gemm_alg = staging + n_jobs * tc * F * esz + sum(((r_eff[(l, k)] + 15) // 16 * 16) * F * 2 + F * 4
                                                     for l, k, _ in jobs)
    dec_alg = stream_total + kv_bytes + sum(((r_eff[(l, k)] + 15) // 16 * 16) * F * 2 + F * 4
                                            for l, k, _ in jobs)
    med = lambda v: float(np.median(v)) * 1e-3
    STAGE1, STAGE2 = "prep_kernel (decode stage 1)", "restore_kernel (decode stage 2)"
    FUSED = "restore_kernel (fused decode)"
    if pipe is None:
        # the step's kernels: encode and the decode's two stages (timed per
        # stage after the steps); the fused schedule is reported beside them
        kern = {"encode_kernel": (enc_alg, med(enc_ms)),
                STAGE1: (prep_alg, med(prep_ms)), STAGE2: (gemm_alg, med(gemm_ms))}
        extra = {FUSED: (dec_alg, med(fused_ms))}
        timed_in = {STAGE1: "two-stage decode loop after the timed steps",
                    STAGE2: "two-stage decode loop after the timed steps",
                    FUSED: "fused-schedule decode loop after the timed steps"}
    else:   # two streams: stage times overlap; report the pipeline as one
        kern = {"encode_kernel": (enc_alg, med(enc_ms)),
                "prep_kernel + restore_kernel (two streams)": (dec_alg, med(dec_ms))}
        extra, timed_in = {}, {}
    # the dominant kernel of the timed step (longest per launch)
    dominant = max(kern, key=lambda k: kern[k][1])
    kern.update(extra)
    enc_t, dec_t = med(enc_ms), med(dec_ms)

    def roof(name):
        alg, t = kern[name]
        per_launch_t = t / n_launch
        ach = alg / n_launch / per_launch_t / 1e9
        r = {"kernel": name, "achieved": round(ach, 1), "frac": round(ach / HBM_PEAK_GBPS, 4),
             "alg_bytes_per_launch": int(alg / n_launch), "us_per_launch": round(per_launch_t * 1e6, 2),
             "launches_per_call": n_launch, "traffic": measured_traffic(name, args.workload)}
        if name in timed_in:
            r["timed_in"] = timed_in[name]
        return r

    flops = sum(2 * F * r_eff[(l, k)] * tc for l, k, _ in jobs)

    # --- compression ratio (host zlib on a sample of streams; not timed)
    host_streams = sbuf.cpu().numpy()
    samp = list(range(0, n_jobs, max(1, n_jobs // 8)))
    raw_s = len(samp) * T * F * esz
    st_s = sum(sizes[i] for i in samp)
    z_s = sum(len(K.kvtc_deflate(host_streams[offs[i]:offs[i] + sizes[i]].tobytes(), 6)) for i in samp)

    result = {
        "metric": "KV encode/decode GB/s (bf16 KV) and % of roofline, Llama-3.1-8B shape 8K tok",
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {n_jobs} tensors x {T} tokens x {F} "
                               f"features {w.dtype}, s={w.sink} w={w.window} G={w.group} "
                               f"{w.bits_per_value} bit/value, encode+decode per step"
                               + (", paged 16-token blocks, two-stream decode" if w.paged else ""),
                   "layers": w.n_layers, "requests": R, "tokens": T, "features": F},
        "encode_GBps": round(kv_bytes / enc_t / 1e9, 2),
        "decode_GBps": round(kv_bytes / dec_t / 1e9, 2),
        "encode_ms": round(enc_t * 1e3, 4),
        "decode_ms": round(dec_t * 1e3, 4),
        "decode_path": {"schedule": "two-stage pipeline" if pipe is not None else "two-stage",
                        "achieved": round(dec_alg / dec_t / 1e9, 1),
                        "frac": round(dec_alg / dec_t / 1e9 / HBM_PEAK_GBPS, 4)},
        "sustained": {"steps": n_sus, "measured": "last 50 steps, HIP events",
                      "ms_per_step": round(float(np.median(sus_enc + sus_dec)), 4),
                      "value": round(kv_bytes / (float(np.median(sus_enc + sus_dec)) * 1e-3) / 1e9, 2),
                      "encode": {"us_per_launch": round(med(sus_enc) / n_launch * 1e6, 2),
                                 "frac": round(enc_alg / med(sus_enc) / 1e9 / HBM_PEAK_GBPS, 4)},
                      "decode_path": {"us_per_launch": round(med(sus_dec) / n_launch * 1e6, 2),
                                      "frac": round(dec_alg / med(sus_dec) / 1e9 / HBM_PEAK_GBPS, 4)}},
        "encode_centred": None if cen_ms is None else {
            "us_per_launch": round(med(cen_ms) / n_launch * 1e6, 2),
            "frac": round(enc_alg / med(cen_ms) / 1e9 / HBM_PEAK_GBPS, 4),
            "timed_in": "kvtc_encode of a copy of the codec with every slot centred, after the timed steps"},
        "decode_alone": {"schedule": "two-stage pipeline" if pipe is not None else "two-stage",
                         "achieved": round(dec_alg / med(alone_ms) / 1e9, 1),
                         "frac": round(dec_alg / med(alone_ms) / 1e9 / HBM_PEAK_GBPS, 4),
                         "timed_in": "the step's decode call in a loop of its own after the timed steps"},
        "roofline": dict(bound="hbm", peak=HBM_PEAK_GBPS, unit="GB/s", **roof(dominant)),
        "roofline_other": [roof(k) for k in kern if k != dominant],
        "mfma_flops_per_call": flops,
        "copy_GBps": round(copy_gbps, 1),
        "compression": {"raw_over_stream": round(raw_s / st_s, 3),
                        "raw_over_deflate": round(raw_s / z_s, 3),
                        "r_eff": sorted(set(r_eff.values()))},
        "calibration_s": None if args.load_artifact else round(calib_s, 1),
    }
    if not args.core_only:
        result["lossless"] = lossless_stage(K, codec, jobs, sizes, offs, sbuf, T, F, esz, dev, stream,
                                            args.steps, raw_s / z_s)
    if pipe is not None:
        result["pipeline"] = pipe.overlap(stream)
    elif not args.core_only:
        result["online_encode"] = online_encode(K, codec, jobs, sizes, offs, T, F, dev, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(codec, w, jobs[: args.cpu_sample], xs, K)
    print(json.dumps(result), flush=True)


class Pipeline:
    """Layer-by-layer decode on two streams: stage 1 (unpack, stream U) of
    later layers overlaps stage 2 (restore, stream R) of layer l; nbuf staging
    buffers and workspaces rotate between layers, so stage 1 runs up to
    nbuf - 1 layers ahead of stage 2."""

    def __init__(self, K, codec, w, jobs, dec_jobs, dev, nbuf=2):
        import torch
        self.K, self.codec, self.torch = K, codec, torch
        self.layers = []
        for l in range(w.n_layers):
            self.layers.append([dj for (jl, _, _), dj in zip(jobs, dec_jobs) if jl == l])
        self.nst = max(codec.staging_bytes(js) for js in self.layers)
        self.nbuf = max(2, min(nbuf, len(self.layers)))
        self.staging = [torch.empty(self.nst, dtype=torch.uint8, device=dev) for _ in range(self.nbuf)]
        self.nj = max(len(js) for js in self.layers)
        self.ws = [torch.zeros(K.kvtc_workspace_bytes(self.nj) // 4, dtype=torch.int32, device=dev)
                   for _ in range(self.nbuf)]
        self.su, self.sr = torch.cuda.Stream(), torch.cuda.Stream()
        L = len(self.layers)
        self.ev_u = [torch.cuda.Event() for _ in range(L)]
        self.ev_r = [torch.cuda.Event() for _ in range(L)]

    def run(self, stream):
        torch, K = self.torch, self.K
        start = torch.cuda.Event()
        start.record(stream)
        self.su.wait_event(start)
        self.sr.wait_event(start)
        for l, js in enumerate(self.layers):
            b = l % self.nbuf
            if l >= self.nbuf:
                self.su.wait_event(self.ev_r[l - self.nbuf])   # staging buffer b is free again
            self.codec.decode_unpack(js, K.KVTC_BF16, self.staging[b], self.nst, self.ws[b], self.su)
            self.ev_u[l].record(self.su)
            self.sr.wait_event(self.ev_u[l])
            self.codec.decode_restore(js, K.KVTC_BF16, self.staging[b], self.nst, self.ws[b], self.sr)
            self.ev_r[l].record(self.sr)
        stream.wait_event(self.ev_r[-1])
        stream.wait_stream(self.su)

    def check(self):
        for b in range(self.nbuf):
            st = self.K.kvtc_read_device_status(self.ws[b], self.nj, None)
            if np.any(st != 0):
                raise SystemExit(f"pipeline status errors: {st}")

    def overlap(self, stream, reps=3):
        """overlap = (unpack time + restore time, back to back on one stream)
        / (two-stream pipelined time)."""
        torch, K = self.torch, self.K
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        seq = []
        for _ in range(reps):
            e[0].record(stream)
            for js in self.layers:
                self.codec.decode_unpack(js, K.KVTC_BF16, self.staging[0], self.nst, self.ws[0], stream)
            e[1].record(stream)
            for js in self.layers:
                self.codec.decode_unpack(js, K.KVTC_BF16, self.staging[0], self.nst, self.ws[0], stream)
                self.codec.decode_restore(js, K.KVTC_BF16, self.staging[0], self.nst, self.ws[0], stream)
            e[2].record(stream)
            torch.cuda.synchronize()
            t_u = e[0].elapsed_time(e[1])
            seq.append((t_u, e[1].elapsed_time(e[2]) - t_u))
        t_u, t_r = np.median(np.array(seq), axis=0)
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(reps):
            p0.record(stream)
            self.run(stream)
            p1.record(stream)
            torch.cuda.synchronize()
            times.append(p0.elapsed_time(p1))
        t_p = float(np.median(times))
        # the same layers each decoded by one fused-schedule call (status
        # words only: no staging), back to back on one stream
        nw = K.kvtc_workspace_bytes(self.nj)
        tf = []
        for _ in range(reps):
            p0.record(stream)
            for js in self.layers:
                self.codec.decode(js, K.KVTC_BF16, self.ws[0], nw, stream)
            p1.record(stream)
            torch.cuda.synchronize()
            tf.append(p0.elapsed_time(p1))
        self.check()
        return {"staging_buffers": self.nbuf, "unpack_ms": round(float(t_u), 4),
                "restore_ms": round(float(t_r), 4), "pipelined_ms": round(t_p, 4),
                "overlap": round(float(t_u + t_r) / t_p, 3),
                "layer_fused_ms": round(float(np.median(tf)), 4)}


def lossless_stage(K, codec, jobs, sizes, offs, sbuf, T, F, esz, dev, stream, reps, deflate_ratio):
    """The GPU lossless stage over every stream of the step: one
    kvtc_lossless_encode call (streams -> containers) and one
    kvtc_lossless_decode call (containers -> streams), timed with events;
    the decoded streams must equal the originals byte for byte. Throughput is
    stream bytes per second; the ratio is raw KV bytes over container bytes,
    beside host zlib's on the sampled streams."""
    import torch
    n = len(jobs)
    bounds = [codec.lossless_bound(l, k, T) for l, k, _ in jobs]
    coff = np.cumsum([0] + [(b + 255) // 256 * 256 for b in bounds])
    cbuf = torch.zeros(int(coff[-1]), dtype=torch.uint8, device=dev)
    back = torch.zeros_like(sbuf)
    ej = [K.make_job(l, k, T, sbuf.data_ptr() + int(offs[i]), cbuf.data_ptr() + int(coff[i]), bounds[i],
                     src_capacity=sizes[i]) for i, (l, k, _) in enumerate(jobs)]
    n_e = codec.lossless_workspace_bytes(ej, True)
    wse = torch.zeros(n_e, dtype=torch.uint8, device=dev)
    dj = [K.make_job(l, k, T, cbuf.data_ptr() + int(coff[i]), back.data_ptr() + int(offs[i]), sizes[i],
                     src_capacity=bounds[i]) for i, (l, k, _) in enumerate(jobs)]
    n_d = codec.lossless_workspace_bytes(dj, False)
    wsd = torch.zeros(n_d, dtype=torch.uint8, device=dev)

    def timed(fn):
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3

    t_enc = timed(lambda: codec.lossless_encode(ej, wse, n_e, stream))
    if np.any(K.kvtc_read_device_status(wse, n, stream) != 0):
        raise SystemExit("device status errors in the lossless encode")
    csizes = K.kvtc_lossless_sizes(wse, n, stream)
    t_dec = timed(lambda: codec.lossless_decode(dj, wsd, n_d, stream))
    if np.any(K.kvtc_read_device_status(wsd, n, stream) != 0):
        raise SystemExit("device status errors in the lossless decode")
    for i in range(n):
        a, b = int(offs[i]), int(offs[i]) + sizes[i]
        if not torch.equal(sbuf[a:b], back[a:b]):
            raise SystemExit(f"lossless round trip differs on tensor {i}")
    st_bytes, c_bytes = int(sum(sizes)), int(csizes.sum())
    raw = n * T * F * esz
    return {"encode_ms": round(t_enc * 1e3, 4), "decode_ms": round(t_dec * 1e3, 4),
            "encode_stream_GBps": round(st_bytes / t_enc / 1e9, 2),
            "decode_stream_GBps": round(st_bytes / t_dec / 1e9, 2),
            "stream_bytes": st_bytes, "container_bytes": c_bytes,
            "raw_over_stream": round(raw / st_bytes, 3), "raw_over_container": round(raw / c_bytes, 3),
            "raw_over_deflate_sample": round(deflate_ratio, 3), "round_trip": "exact"}


def online_encode(K, codec, jobs, sizes, offs, T, F, dev, stream, hidden=4096, reps=3, enc_wgs=32):
    """Layer-by-layer encode overlapped with KV production: a producer (a bf16
    GEMM of [T, hidden] states by a [hidden, F] projection per tensor, torch,
    standing in for the model's K and V projections) writes layer l + 1 on
    one stream while kvtc_encode compresses layer l on another. Reported: the
    producer alone, the per-layer encodes alone and back to back, the two
    streams together (the encode with its full persistent grid, and capped
    at enc_wgs workgroups so that most of the chip stays with the producer),
    and the share of the encode time the overlap hides."""
    import torch
    layers = sorted({l for l, _, _ in jobs})
    idx = {l: [i for i, (jl, _, _) in enumerate(jobs) if jl == l] for l in layers}
    g = torch.Generator(device=dev).manual_seed(3)
    h = torch.randn((T, hidden), generator=g, device=dev).to(torch.bfloat16)
    wts = (torch.randn((len(jobs), hidden, F), generator=g, device=dev) * hidden ** -0.5).to(torch.bfloat16)
    kv = torch.empty((len(jobs), T, F), dtype=torch.bfloat16, device=dev)
    sbuf = torch.empty(int(offs[-1]), dtype=torch.uint8, device=dev)
    ljobs = {l: [K.make_job(jobs[i][0], jobs[i][1], T, kv[i], sbuf.data_ptr() + int(offs[i]), sizes[i])
                 for i in idx[l]] for l in layers}
    ws = {l: torch.zeros(K.kvtc_workspace_bytes(len(idx[l])) // 4, dtype=torch.int32, device=dev)
          for l in layers}
    sp, se = torch.cuda.Stream(), torch.cuda.Stream()
    ev = {l: torch.cuda.Event() for l in layers}

    def produce(l):
        for i in idx[l]:
            torch.matmul(h, wts[i], out=kv[i])

    def timed(fn):
        t = []
        for _ in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b))
        return float(np.median(t[1:]))

    def pipelined(p_s, e_s):
        start = torch.cuda.Event()
        start.record(stream)
        p_s.wait_event(start)
        e_s.wait_event(start)
        for l in layers:
            with torch.cuda.stream(p_s):
                produce(l)
                ev[l].record(p_s)
            e_s.wait_event(ev[l])
            codec.encode(ljobs[l], ws[l], e_s)
        stream.wait_stream(e_s)
        stream.wait_stream(p_s)

    def capped(fn, cap):
        old = os.environ.get("KVTC_MAX_WORKGROUPS")
        os.environ["KVTC_MAX_WORKGROUPS"] = str(cap)
        try:
            return fn()
        finally:
            if old is None:
                del os.environ["KVTC_MAX_WORKGROUPS"]
            else:
                os.environ["KVTC_MAX_WORKGROUPS"] = old

    t_prod = timed(lambda: [produce(l) for l in layers])
    t_enc = timed(lambda: [codec.encode(ljobs[l], ws[l], stream) for l in layers])
    t_seq = timed(lambda: [(produce(l), codec.encode(ljobs[l], ws[l], stream)) for l in layers])
    t_pipe = timed(lambda: pipelined(sp, se))
    t_pipe_m = capped(lambda: timed(lambda: pipelined(sp, se)), enc_wgs)
    for l in layers:
        if np.any(K.kvtc_read_device_status(ws[l], len(idx[l]), stream) != 0):
            raise SystemExit("device status errors in the online encode")
    best = min(t_pipe, t_pipe_m)
    return {"layers": len(layers), "producer": f"bf16 GEMM [{T} x {hidden}] x [{hidden} x {F}] per tensor",
            "producer_ms": round(t_prod, 4), "encode_ms": round(t_enc, 4), "sequential_ms": round(t_seq, 4),
            "pipelined_ms": round(t_pipe, 4),
            f"pipelined_encode_{enc_wgs}_workgroups_ms": round(t_pipe_m, 4),
            "overlap": round(t_seq / best, 3), "encode_hidden": round((t_seq - best) / t_enc, 3)}


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs recorded in profiles/traffic.json, if they were taken on
    this workload with the kernel source as it is now (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    csrc = os.path.join(ROOT, "kv_cache_transform_amd", "csrc")
    try:
        with open(path) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for name in KERNEL_SOURCES:
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
        digest = h.hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernels_sha256") != digest or rec.get("workload") != workload:
        return None
    k = rec.get("per_launch_bytes", {}).get(kernel)
    return int(k) if k is not None else None


def cpu_baseline(codec, w, sample, xs, K, budget_s=12.0):
    """The CPU oracle, untouched, timed on host copies of the same tensors
    (tensors in order until about budget_s seconds of work)."""
    import oracle.kvtc_oracle as O
    from threadpoolctl import threadpool_info

    art = O.parse_artifact(codec.save())
    p = art.params
    T, F = w.n_tokens, w.features
    t_enc = t_dec = 0.0
    done = []
    for i, (l, k, _) in enumerate(sample):
        if t_enc + t_dec > budget_s:
            break
        store = xs[i].cpu().numpy()
        store = store.view(np.uint16) if store.dtype == np.int16 else store
        t = time.perf_counter()
        er = O.encode(store, p, art.slots[(l, k)], l, k)
        t_enc += time.perf_counter() - t
        t = time.perf_counter()
        O.decode(er.stream, p, art.slots[(l, k)], l, k, T, O.DTYPE_BF16)
        t_dec += time.perf_counter() - t
        done.append((l, k))
    kv = len(done) * T * F * w.elem_bytes
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(kv / (t_enc + t_dec) / 1e9, 4), "unit": "GB/s",
            "cores": int(threads), "kind": "oracle",
            "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model,
            "encode_GBps": round(kv / t_enc / 1e9, 4), "decode_GBps": round(kv / t_dec / 1e9, 4),
            "sample": f"{len(done)} of {w.n_tensors} tensors ({len(done)} x {T} x {F} "
                      f"{w.dtype}), encode + decode, same artifact, about {budget_s:.0f} s"}


if __name__ == "__main__":
    main()
