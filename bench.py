"""Benchmark of the QSGD compressor hot path on one MI355X.

A step is one encode (quantize + Elias-omega stream, one pass over v) and one
decode (parse + dequantize) of a synthetic gradient shaped like the pages'
workloads; by default the ResNet-152-sized one (n = 60,192,808 fp32, buckets
d = 4096, s = 64), --config 1..5 picks another. Inputs are resident in HBM.
Several copies of the input and output buffers are rotated, and a 512 MiB
buffer is overwritten before each timed call (outside the timed region), so
that no call finds its input in the 256 MB Infinity Cache -- decode included,
which would otherwise read the stream the encode has just written.

Prints one JSON line: value = whole-job round-trip throughput 4n bytes of fp32
gradient / (encode + decode time) in GB/s, plus per-direction rates (median,
p10, p90) and HBM fractions, bits per coordinate, the roofline object of the
dominant single kernel (the decode call is one kernel launch) with its
counter-measured HBM traffic and VALU-issue fraction where the committed
counters match the sources, and the oracle's rate on one pinned host core.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
VALU_PEAK_GIPS = 256 * 4 * 2.4e9 / 4 / 1e9  # wave64 VALU instructions per s: 614.4 G


def traffic_file(config: int) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_c{config}.json")


def kernel_source_hash() -> str:
    """Hash of the HIP sources: counter-derived traffic is only reported for the
    kernels it was measured on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_sgd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_counters(config: int, kernel: str):
    """The committed counter record of `kernel` on this config (HBM bytes and
    VALU instructions per launch), or {} if it is missing or was taken on other
    kernel sources."""
    try:
        with open(traffic_file(config)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    if rec.get("source_hash") != kernel_source_hash():
        return {}
    return rec.get("kernels", {}).get(kernel, {})


def cpu_identity():
    """Host CPU model and core counts (the CPU baseline's context)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count()
    return {"cpu_model": model, "nproc": avail, "cpu_count": os.cpu_count()}


def copy_calibration(mbytes: int, reps: int):
    """A plain device-to-device copy of known size (the counter calibration run
    for FETCH_SIZE / WRITE_SIZE)."""
    import torch
    n = mbytes * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 4 * n, "reps": reps}), flush=True)


def cpu_baseline(w, max_coords: int, reps: int = 3):
    """The oracle (single-threaded C, as it stands) on the first whole buckets
    of the workload (all of it by default): quantize + encode + decode, median of
    `reps` runs, with this process pinned to one host core (the first it may
    use) for the duration."""
    import numpy as np

    import oracle
    ident = cpu_identity()
    try:
        prev = os.sched_getaffinity(0)
        core = min(prev)
        os.sched_setaffinity(0, {core})
    except (AttributeError, OSError):
        prev, core = None, None
    if w.seg_len is not None:  # ragged batch: the whole batch
        m = w.n
        bst = oracle.ragged_buckets(w.seg_len, w.d)
    else:
        m = min(w.n, (max_coords // w.d) * w.d) if max_coords > 0 else w.n
        bst = oracle.uniform_buckets(m, w.d)
    v = np.ascontiguousarray(w.v[:m])
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        lev, nrm = oracle.quantize(v, bst, w.s, w.seed)
        words, offs, nbits = oracle.encode(lev, nrm, bst, w.s)
        rc, vh = oracle.decode(words, offs, bst, w.s)
        times.append(time.perf_counter() - t0)
        assert rc == oracle.OK
    if prev is not None:
        os.sched_setaffinity(0, prev)
    t = sorted(times)[len(times) // 2]
    return {"value": round(4.0 * m / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{m} coordinates ({len(bst) - 1} buckets) of the same gradient; "
                      f"quantize+encode+decode, median of {reps} runs, {t:.2f} s each",
            "pinned_core": core, **ident}


def variant_leg(q, torch, args, v, lay, n, s, d, seed, nb, stream, nbits_omega, code, norm, flush):
    """The same workload with another record code (Elias gamma) or bucket scale
    (max-norm, the QSGDinf reading), through qsgd_encode_ex / qsgd_decode_ex:
    call times on the launch stream (the same cache flush before each), bits per
    coordinate, and the algorithmic-bytes HBM fractions, next to the default's."""
    dev = v.device
    G = code
    ragged = lay is not None
    cap = lay.capacity_words(s, G) if ragged else q.encode_capacity_words(n, s, d, G)
    out = torch.empty(cap, dtype=torch.int64, device=dev)
    bits = torch.empty(1, dtype=torch.int64, device=dev)
    offs = torch.empty(nb + 1, dtype=torch.int64, device=dev)
    vh = torch.empty(n, dtype=torch.float32, device=dev)

    def enc():
        if ragged:
            q.encode_ragged(v, lay, s, seed, out=out, out_bits=bits, offsets=offs, code=G, norm=norm)
        else:
            q.encode(v, s, d, seed, out=out, out_bits=bits, offsets=offs, code=G, norm=norm)

    def dec():
        if ragged:
            q.decode_ragged(out, offs, lay, s, v_hat=vh, code=G)
        else:
            q.decode(out, offs, n, s, d, v_hat=vh, code=G)

    for _ in range(2):
        enc()
        dec()
    torch.cuda.synchronize()
    steps = max(1, args.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        flush()
        ev[i][0].record(stream)
        enc()
        ev[i][1].record(stream)
        flush()
        ev[i][2].record(stream)
        dec()
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    e_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    d_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    nbits = int(bits.item())
    alg = 4.0 * n + nbits / 8.0 + 8.0 * (nb + 1)
    return {"encode_ms_avg": round(e_ms, 4), "decode_ms_avg": round(d_ms, 4),
            "round_trip_GBps_fp32": round(4.0 * n / ((e_ms + d_ms) * 1e-3) / 1e9, 2),
            "bits_per_coord": round(nbits / n, 4), "bits_vs_default": round(nbits / nbits_omega, 4),
            "encode_hbm_frac": round(alg / (e_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "decode_hbm_frac": round(alg / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def decode_accumulate_leg(q, wl, torch, args, v0, n, s, d, seed, nb, stream, flush):
    """Decode-accumulate of k workers' streams (worker 0: the config's gradient)
    into one fp32 buffer, timed with HIP events on the launch stream. Algorithmic
    HBM bytes (the least any implementation moves): the k streams and offset
    tables read, acc read and written once."""
    k = args.acc_streams
    dev = v0.device
    words, offs, nbits = [], [], 0
    for j in range(k):
        vj = v0 if j == 0 else torch.from_numpy(wl.peer_gradient(args.config, j)).to(dev)
        o, b, f = q.encode(vj, s, d, seed + j)
        words.append(o)
        offs.append(f)
        nbits += int(b.item())
        del vj
    acc = torch.zeros(n, dtype=torch.float32, device=dev)
    for _ in range(2):
        q.decode_accumulate(words, offs, n, s, d, acc)
    torch.cuda.synchronize()
    steps = max(1, args.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        flush()
        ev[i][0].record(stream)
        q.decode_accumulate(words, offs, n, s, d, acc)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    avg = sum(ms) / steps
    alg = 8.0 * n + nbits / 8.0 + 8.0 * k * (nb + 1)
    return {"streams": k, "ms_median": round(ms[len(ms) // 2], 4), "ms_avg": round(avg, 4),
            "decoded_GBps_fp32": round(4.0 * n * k / (avg * 1e-3) / 1e9, 2),
            "hbm_GBps_algorithmic": round(alg / (avg * 1e-3) / 1e9, 2),
            "hbm_frac": round(alg / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes": round(alg)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--cpu-sample", type=int, default=0, help="coordinates for the oracle (0: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the Elias-gamma and max-norm legs")
    ap.add_argument("--acc-streams", type=int, default=4,
                    help="streams of the decode-accumulate measurement (configs 2, 3; 0: skip)")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="MiB read (or overwritten) before each timed call, outside the timed region (0: none)")
    ap.add_argument("--flush-kind", choices=["read", "write"], default="read",
                    help="how the cache flush before each timed call evicts the inputs: "
                         "by reading the flush buffer, or by overwriting it")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="only run a plain copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.copy_calib_mb:
        copy_calibration(args.copy_calib_mb, max(1, args.steps))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the compressor needs no second GPU); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_sgd_amd as q
    from quantized_sgd_amd import workloads as wl

    w = wl.CONFIGS[args.config]()
    n, s, d, seed = w.n, w.s, w.d, w.seed
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R = max(1, args.rotate)
    host = torch.from_numpy(w.v)
    vs = [host.to(dev) for _ in range(R)]
    ragged = w.seg_len is not None
    lay = q.RaggedLayout(w.seg_len, d) if ragged else None
    nb = lay.nb if ragged else q.num_buckets(n, d)
    cap = lay.capacity_words(s) if ragged else q.encode_capacity_words(n, s, d)
    outs = [torch.empty(cap, dtype=torch.int64, device=dev) for _ in range(R)]
    bits = [torch.empty(1, dtype=torch.int64, device=dev) for _ in range(R)]
    offs = [torch.empty(nb + 1, dtype=torch.int64, device=dev) for _ in range(R)]
    vhs = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)]
    stream = torch.cuda.current_stream()

    def enc(r):
        if ragged:
            q.encode_ragged(vs[r], lay, s, seed, out=outs[r], out_bits=bits[r], offsets=offs[r])
        else:
            q.encode(vs[r], s, d, seed, out=outs[r], out_bits=bits[r], offsets=offs[r])

    def dec(r):
        if ragged:
            q.decode_ragged(outs[r], offs[r], lay, s, v_hat=vhs[r])
        else:
            q.decode(outs[r], offs[r], n, s, d, v_hat=vhs[r])

    flush_buf = torch.empty(max(1, args.flush_mb) * (1 << 20) // 4, dtype=torch.float32, device=dev) \
        if args.flush_mb else None

    def flush():
        # evict the inputs from the caches (outside the timed region) by reading a
        # buffer larger than the 256 MB Infinity Cache: dirty lines are written
        # back here, and the timed call finds the caches holding clean lines only.
        # Overwriting the buffer instead leaves up to 256 MB of its dirty lines for
        # the timed call to write back.
        if flush_buf is not None:
            if args.flush_kind == "read":
                flush_buf.sum(dtype=torch.float32)
            else:
                flush_buf.fill_(0.0)

    for i in range(args.warmup):
        enc(i % R)
        dec(i % R)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        r = i % R
        flush()
        ev[i][0].record(stream)
        enc(r)
        ev[i][1].record(stream)
        flush()
        ev[i][2].record(stream)
        dec(r)
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    enc_ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    dec_ms = sorted(e[2].elapsed_time(e[3]) for e in ev)
    pct = lambda a, f: a[min(len(a) - 1, int(round(f * (len(a) - 1))))]
    enc_avg = sum(enc_ms) / K
    dec_avg = sum(dec_ms) / K
    ms_per_step = (t1 - t0) * 1e3 / K
    nbits = int(bits[0].item())
    gbytes = 4.0 * n / 1e9
    # algorithmic bytes per launch: encode reads v, writes the stream and offsets;
    # decode reads the stream and offsets, writes v_hat
    side = 8.0 * (nb + 1)
    enc_bytes = 4.0 * n + nbits / 8.0 + side
    dec_bytes = nbits / 8.0 + side + 4.0 * n
    enc_gbps = enc_bytes / (enc_avg * 1e-3) / 1e9
    dec_gbps = dec_bytes / (dec_avg * 1e-3) / 1e9

    def roofline(kind, t_ms, alg_bytes):
        c = measured_counters(args.config, kind)
        ach = alg_bytes / (t_ms * 1e-3) / 1e9
        out = {"bound": "hbm", "kernel": c.get("kernel_names", [kind]), "achieved": round(ach, 2),
               "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
               "traffic": c.get("hbm_bytes_per_launch"), "algorithmic_bytes": round(alg_bytes),
               "launch_ms_avg": round(t_ms, 4)}
        valu = c.get("valu_insts_per_launch")
        if valu is not None:
            out["valu"] = {"insts_per_launch": valu, "peak_ginsts_per_s": VALU_PEAK_GIPS,
                           "frac": round(valu / (t_ms * 1e-3) / (VALU_PEAK_GIPS * 1e9), 4)}
        return out

    res = {
        "metric": "QSGD encode/decode GB/s of fp32 gradient on 1 MI355X; % HBM peak; bits/coord",
        "value": round(gbytes / ((enc_avg + dec_avg) * 1e-3), 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "n": n, "d": d, "s": s, "buckets": nb,
                   "input_copies_rotated": R, "flush_mb_between_calls": args.flush_mb,
                   "flush_kind": args.flush_kind},
        "encode_ms": {"median": round(pct(enc_ms, 0.5), 4), "p10": round(pct(enc_ms, 0.1), 4),
                      "p90": round(pct(enc_ms, 0.9), 4), "avg": round(enc_avg, 4)},
        "decode_ms": {"median": round(pct(dec_ms, 0.5), 4), "p10": round(pct(dec_ms, 0.1), 4),
                      "p90": round(pct(dec_ms, 0.9), 4), "avg": round(dec_avg, 4)},
        "encode_GBps_fp32": round(gbytes / (enc_avg * 1e-3), 2),
        "decode_GBps_fp32": round(gbytes / (dec_avg * 1e-3), 2),
        "encode_hbm_frac": round(enc_gbps / HBM_PEAK_GBPS, 4),
        "decode_hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "bits_per_coord": round(nbits / n, 4),
        "compression_vs_fp32": round(32.0 * n / nbits, 3),
        "compression_vs_fp32_with_offsets": round(32.0 * n / (nbits + 64.0 * (nb + 1)), 3),
        # the decode call is a single kernel launch; the encode call is two
        # (pass 1 and the pass-2 gather) and is reported beside it
        "roofline": roofline("decode", dec_avg, dec_bytes),
        "encode_call_roofline": roofline("encode", enc_avg, enc_bytes),
    }
    if not args.no_variants:
        res["gamma"] = variant_leg(q, torch, args, vs[0], lay, n, s, d, seed, nb, stream, nbits,
                                   q.GAMMA, q.L2, flush)
        res["maxnorm"] = variant_leg(q, torch, args, vs[0], lay, n, s, d, seed, nb, stream, nbits,
                                     q.OMEGA, q.MAXNORM, flush)
    if args.acc_streams and args.config in (2, 3) and not ragged:
        res["decode_accumulate"] = decode_accumulate_leg(q, wl, torch, args, vs[0], n, s, d, seed, nb, stream,
                                                         flush)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
