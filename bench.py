"""Benchmark of the groupwise low-bit linear hot path on one MI355X.

One step = one pass of the hot path over the headline workloads:
  * decode (qmv): M=1, K=N=4096, group 64, fp16 activations, bits 1..7 --
    the Llama-3.1-8B-shaped decode linears at K=N=4096;
  * batched (qmm, MFMA): M=128, bits 4, group 128, bf16, (K, N) = (4096, 14336)
    and (14336, 4096).
Inputs are seeded synthetic tensors (no checkpoints), already resident in GPU
memory when timing starts; weights are quantized and packed on the GPU before
timing (quantization is one-off, not on the decode path).  To keep the
256 MB Infinity Cache from serving repeated weights, every case rotates
through its own set of weight copies of >= 1 GiB, so every launch (in the
per-kernel loops as in the steps) reads weights that are not cached.

Beside the decode timings the benchmark measures the single-launch floor of
the device: a plain streaming read of the same byte count in one launch (the
best of 1, 2, 4 and 8 loads per thread, over the same kind of rotation) and
the latency of one dependent load from HBM (a pointer chase), since at a few
MB per call launch and memory latency, not bandwidth, bound any one kernel.

Printed: one JSON line.  `value` is the decode kernels' achieved algorithmic
HBM bandwidth over bits 1..7 (sum of bytes / sum of kernel times); per-bit
microseconds and GB/s and the batched kernel's TFLOP/s are extra fields.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from bit_groupwise_weight_amd import probe  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
MFMA_I8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA
ROTATE_BYTES = 1 << 30

# HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE passes (and
# the MFMA kernel's MfmaUtil) whose commands and scaling are recorded in
# profiles/ (FETCH_SIZE x 2.000, WRITE_SIZE x 1.000, from a plain 256 MiB
# copy).  They describe the
# kernel sources whose sha256 prefix is `src_hash`; for any other sources bench
# reports traffic as null.
MEASURED_TRAFFIC = {
    "src_hash": "82f3c1b5a2a23a45",
    "qmv_bits1to7_bytes": 67126704,
    "qmm_bytes": {"4096x14336": 72810909, "14336x4096": 95351564},
    # rocprofv3 MfmaUtil (%) of the main MFMA kernel per shape
    "qmm_mfma_util": {"4096x14336": 19.59, "14336x4096": 19.92},
    # HBM bytes per launch of the int8-activation linear per (K x N) shape
    "a8_bytes": {"4096x14336": 44670492, "14336x4096": 52536189},
}


def kernel_source_hash() -> str:
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "bit_groupwise_weight_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=50,
                    help="launches per kernel in the per-kernel timing loops")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-reps", type=int, default=30)
    ap.add_argument("--no-decode-layer", action="store_true",
                    help="skip the decoder-layer section (its q-proj launches share the kernel "
                         "and grid of the b=4 decode case, which a kernel trace would mix up)")
    ap.add_argument("--no-eager", action="store_true",
                    help="skip the one-call-per-launch timing (profiling runs: only graph launches)")
    ap.add_argument("--no-a8", action="store_true",
                    help="skip the activation-quantized variant (int8 dynamic activations)")
    ap.add_argument("--no-floor", action="store_true",
                    help="skip the streaming-read and load-latency measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy (a kernel of known "
                         "traffic, to scale hardware byte counters)")
    ap.add_argument("--all-configs", action="store_true",
                    help="after the timed steps, time every workload configuration (127 cases, "
                         "each with its own rotation) and the single-launch floor at the wide "
                         "decode shapes; adds the field all_configs (not part of value)")
    ap.add_argument("--only-configs", default="",
                    help="with --all-configs: comma-separated workload keys to run (single, "
                         "llama8b, llama_small, batched, mixed); default all")
    return ap.parse_args()


def qmv_cases():
    from bit_groupwise_weight_amd.workloads import Case
    return [Case(f"llama8b_k4096_n4096_b{b}_g64", 1, 4096, 4096, b, 64, "f16") for b in range(1, 8)]


def qmm_cases():
    from bit_groupwise_weight_amd.workloads import batched_qmm
    return batched_qmm()


def algo_bytes(case) -> int:
    """Bytes the layer must move: packed codes + scales + zeros + x + y (+ bias)."""
    e = {"f32": 4, "f16": 2, "bf16": 2}[case.act]
    b = case.N * case.K * case.bits // 8 + 2 * case.N * (case.K // case.group) * e
    b += case.M * case.K * e + case.M * case.N * e
    if case.bias:
        b += case.N * e
    return b


def prepare(case, copies, dev):
    """Quantize once on the GPU and make `copies` independent copies of the weights."""
    from bit_groupwise_weight_amd import lowbit as lb
    from bit_groupwise_weight_amd.workloads import make_bias, make_weight, make_x
    act = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[case.act]
    W = make_weight(case).to(dev)
    packed, s, z, _ = lb.lowbit_quantize_pack(W, case.bits, case.group, act)
    del W
    x = make_x(case).to(dev)
    b = make_bias(case)
    b = None if b is None else b.to(dev)
    sets = [(packed, s, z)] + [(packed.clone(), s.clone(), z.clone()) for _ in range(copies - 1)]
    ys = [torch.empty((case.M, case.N), dtype=act, device=dev) for _ in range(2)]
    return {"case": case, "sets": sets, "x": x, "bias": b, "ys": ys}


def launch(p, i, stream):
    """One lowbit_linear call on weight copy i (mod copies)."""
    from bit_groupwise_weight_amd import lowbit as lb
    c = p["case"]
    packed, s, z = p["sets"][i % len(p["sets"])]
    lb.lowbit_linear(p["x"], packed, s, z, p["bias"], c.bits, c.group, y=p["ys"][i % 2],
                     stream=stream)


def capture(fn, n, stream):
    """A HIP graph holding fn(0), ..., fn(n-1), captured on a side stream."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream()
        for i in range(n):
            fn(i, s)
    return g


def time_graph(g, replays, per_replay, stream):
    """Microseconds per unit of work: HIP events around `replays` replays of a
    graph holding `per_replay` units, recorded on the replay stream."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(replays):
        g.replay()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * per_replay)


def time_eager(p, reps, stream, prepared=True):
    """Microseconds per call when launched one by one from Python (host-bound):
    through a PreparedLinear per weight copy (weights validated once, as the
    module's eager forward does), or through lowbit_linear (every tensor
    validated on every call)."""
    from bit_groupwise_weight_amd import lowbit as lb
    c = p["case"]
    if prepared:
        calls = [lb.PreparedLinear(pk, s, z, p["bias"], c.bits, c.group) for (pk, s, z) in p["sets"]]
        n = len(calls)

        def one(i):
            calls[i % n](p["x"], y=p["ys"][i % 2], stream=stream)
    else:
        def one(i):
            launch(p, i, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for i in range(3):
        one(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        one(i)
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


# Llama-3.1-8B decoder layer linears (name, N, K), M = 1.
LAYER_SHAPES = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
                ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
LAYER_BITS, LAYER_GROUP = 4, 64


def prepare_a8(case, copies, dev):
    """Weights as prepare(); int8 activation buffers for the quantizer's output."""
    p = prepare(case, copies, dev)
    p["xq"] = torch.empty((case.M, case.K), dtype=torch.int8, device=dev)
    p["ascale"] = torch.empty((case.M,), dtype=torch.float32, device=dev)
    return p


def launch_a8(p, i, stream, quant=True, linear=True):
    """The activation-quantized variant on weight copy i: the per-row int8
    quantizer, then the int8 linear."""
    from bit_groupwise_weight_amd import lowbit as lb
    c = p["case"]
    if quant:
        lb.lowbit_quantize_act_i8(p["x"], p["xq"], p["ascale"], stream=stream)
    if linear:
        packed, s, z = p["sets"][i % len(p["sets"])]
        lb.lowbit_linear_a8(p["xq"], p["ascale"], packed, s, z, p["bias"], c.bits, c.group,
                            y=p["ys"][i % 2], stream=stream)


def activation_quantized(dev, stream, reps):
    """Graph-timed quantizer, linear and whole call at the batched Llama-3.1-8B
    MLP shapes (M=128, bits 4, group 32, bf16)."""
    from bit_groupwise_weight_amd.workloads import activation_quantized as a8_cases
    rows = []
    for c in a8_cases():
        p = prepare_a8(c, copies_for(c), dev)
        torch.cuda.synchronize()
        n = len(p["sets"])
        reps_n = max(2, reps // n + 1)
        t = {}
        for key, kw in (("quant_us", dict(linear=False)), ("linear_us", dict(quant=False)),
                        ("call_us", {})):
            g = capture(lambda i, s, kw=kw: launch_a8(p, i, s, **kw), n, stream)
            t[key] = time_graph(g, reps_n, n, stream)
            del g
        del p
        torch.cuda.empty_cache()
        ops = 2.0 * c.M * c.N * c.K
        tops = ops / (t["linear_us"] * 1e-6) / 1e12
        rows.append({"K": c.K, "N": c.N, "M": c.M, "bits": c.bits, "group": c.group,
                     **{k: round(v, 3) for k, v in t.items()},
                     "TOP_s": round(tops, 2), "frac_i8_peak": round(tops / MFMA_I8_PEAK_TOPS, 4),
                     "TOP_s_call": round(ops / (t["call_us"] * 1e-6) / 1e12, 2)})
        log(f"a8 K={c.K} N={c.N}: quant {t['quant_us']:.2f} us, linear {t['linear_us']:.2f} us "
            f"({tops:.1f} TOP/s), call {t['call_us']:.2f} us")
    return rows


def prepare_layer(copies, dev):
    """One decoder layer's seven linears (seeded N(0, 0.02) weights, quantized on
    the GPU), `copies` independent weight copies, fp16 activations."""
    from bit_groupwise_weight_amd import lowbit as lb
    gen = torch.Generator().manual_seed(1234)
    lin = {}
    for name, N, K in LAYER_SHAPES:
        W = (torch.randn((N, K), generator=gen) * 0.02).to(dev)
        packed, s, z, _ = lb.lowbit_quantize_pack(W, LAYER_BITS, LAYER_GROUP, torch.float16)
        del W
        lin[name] = [(packed, s, z)] + [(packed.clone(), s.clone(), z.clone()) for _ in range(copies - 1)]
    xs = {K: torch.randn((1, K), generator=gen).to(torch.float16).to(dev) for K in (4096, 14336)}
    ys = {name: torch.empty((1, N), dtype=torch.float16, device=dev) for name, N, _ in LAYER_SHAPES}
    return {"lin": lin, "x": xs, "y": ys, "copies": copies}


def layer_bytes() -> int:
    return sum(N * K * LAYER_BITS // 8 + 2 * N * (K // LAYER_GROUP) * 2 + 2 * K + 2 * N
               for _, N, K in LAYER_SHAPES)


def layer_separate(L, i, stream):
    """The seven linears as seven launches."""
    from bit_groupwise_weight_amd import lowbit as lb
    c = i % L["copies"]
    for name, N, K in LAYER_SHAPES:
        packed, s, z = L["lin"][name][c]
        lb.lowbit_linear(L["x"][K], packed, s, z, None, LAYER_BITS, LAYER_GROUP, y=L["y"][name],
                         stream=stream)


def layer_fused(L, i, stream):
    """The same linears as four launches: q/k/v together, o, gate/up together, down."""
    from bit_groupwise_weight_amd import lowbit as lb
    c = i % L["copies"]

    def item(name, K):
        packed, s, z = L["lin"][name][c]
        return (L["x"][K], packed, s, z, None, L["y"][name])

    lb.lowbit_linear_multi([item("q", 4096), item("k", 4096), item("v", 4096)], LAYER_BITS,
                           LAYER_GROUP, stream=stream)
    lb.lowbit_linear_multi([item("o", 4096)], LAYER_BITS, LAYER_GROUP, stream=stream)
    lb.lowbit_linear_multi([item("gate", 4096), item("up", 4096)], LAYER_BITS, LAYER_GROUP,
                           stream=stream)
    lb.lowbit_linear_multi([item("down", 14336)], LAYER_BITS, LAYER_GROUP, stream=stream)


def plain_read_us(byte_counts, dev, stream, reps):
    """Per byte count: the best (microseconds, loads per thread) of a plain
    16-byte streaming read of that many bytes in one launch, rotating over
    >= 1 GiB, graph-timed."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    buf = torch.empty(ROTATE_BYTES + (64 << 20), dtype=torch.uint8, device=dev)
    out = []
    for nb in byte_counts:
        nb16 = (nb + 15) // 16 * 16
        slot = (nb16 + 4095) // 4096 * 4096
        n = max(2, ROTATE_BYTES // slot)
        best = None
        for lpt in (1, 2, 4, 8):
            def fn(i, s, lpt=lpt):
                probe.stream_read(buf[(i % n) * slot:], nb16, lpt, sink, stream=s)
            for i in range(3):
                fn(i, stream)
            g = capture(fn, n, stream)
            us = time_graph(g, max(1, reps // n + 1), n, stream)
            del g
            if best is None or us < best[0]:
                best = (us, lpt)
        out.append(best)
    del buf
    torch.cuda.empty_cache()
    return out


def single_launch_floor(byte_counts, qmv_us, dev, stream, reps):
    """The device's floor for one kernel that reads a few MB: a plain
    streaming read of each byte count in one launch, rotating over >= 1 GiB
    (graph-timed like the decode kernels; best of 1/2/4/8 loads per thread),
    and the latency of one dependent load from HBM (pointer chase over 1 GiB
    with links on distinct 128-byte lines, after a 1 GiB read has flushed the
    caches)."""
    from bit_groupwise_weight_amd import lowbit as lb
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    buf = torch.empty(ROTATE_BYTES + (64 << 20), dtype=torch.uint8, device=dev)
    read_us, read_lpt = [], []
    for nb in byte_counts:
        nb16 = (nb + 15) // 16 * 16
        slot = (nb16 + 4095) // 4096 * 4096
        n = max(2, ROTATE_BYTES // slot)
        best, best_lpt = None, None
        for lpt in (1, 2, 4, 8):
            def fn(i, s, lpt=lpt):
                probe.stream_read(buf[(i % n) * slot:], nb16, lpt, sink, stream=s)
            for i in range(3):
                fn(i, stream)
            g = capture(fn, n, stream)
            us = time_graph(g, max(1, reps // n + 1), n, stream)
            del g
            if best is None or us < best:
                best, best_lpt = us, lpt
        read_us.append(best)
        read_lpt.append(best_lpt)
    # pointer chase: links on distinct random 128-byte lines of a 1 GiB array
    words = ROTATE_BYTES // 4
    hops = 4096
    gen = torch.Generator().manual_seed(5)
    lines = torch.randperm(words // 32, generator=gen)[:hops] * 32
    chain = torch.zeros(words, dtype=torch.int32, device=dev)
    chain[lines.to(dev)] = torch.roll(lines, -1).to(torch.int32).to(dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    start = int(lines[0])

    def chase_us(h):
        probe.stream_read(buf, ROTATE_BYTES, 4, sink, stream=stream)   # flush caches
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        probe.chase(chain, h, start, out, stream=stream)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3

    chase_us(64)
    lat = [(chase_us(hops) - chase_us(64)) / (hops - 64) for _ in range(3)]
    lat_us = sorted(lat)[1]
    del chain, buf
    torch.cuda.empty_cache()
    per_bit = []
    for b, (nb, r, lpt, q) in enumerate(zip(byte_counts, read_us, read_lpt, qmv_us), start=1):
        lower = lat_us + nb / (HBM_PEAK_GBPS * 1e3)
        per_bit.append({"bits": b, "bytes": nb, "stream_read_us": round(r, 3),
                        "stream_read_loads_per_thread": lpt,
                        "stream_read_GB_s": round(nb / (r * 1e-6) / 1e9, 1),
                        "qmv_us": round(q, 3), "qmv_over_stream_read": round(q / r, 3),
                        "latency_plus_peak_transfer_us": round(lower, 3)})
        log(f"floor b={b}: plain read {r:.3f} us ({lpt} loads/thread), qmv {q:.3f} us, "
            f"latency + bytes at 8 TB/s {lower:.3f} us")
    log(f"HBM dependent-load latency: {lat_us:.3f} us")
    tot_read, tot_q = sum(read_us), sum(qmv_us)
    return {"hbm_load_latency_us": round(lat_us, 3),
            "stream_read_total_us": round(tot_read, 3),
            "qmv_total_us": round(tot_q, 3),
            "qmv_frac_of_stream_read": round(tot_read / tot_q, 4),
            "stream_read_GB_s_aggregate": round(sum(byte_counts) / (tot_read * 1e-6) / 1e9, 1),
            "by_bits": per_bit,
            "note": "plain 16-byte streaming read of each decode case's algorithmic byte count "
                    "in one launch (rotating over >= 1 GiB, graph-timed, best of 1/2/4/8 loads "
                    "per thread); latency = pointer chase over 1 GiB on distinct 128-byte lines "
                    "after a 1 GiB read; qmv_frac_of_stream_read = plain-read time / qmv time "
                    "summed over bits 1..7"}


def host_cpu():
    """This host's CPU model and the cores this process may use."""
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
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    return model, nproc


def cpu_baseline(cases, reps, single_reps=3):
    """The CPU oracle's linear (fp64 dequant + matmul) timed on this host: on
    all the threads its BLAS uses (the reported value) and on one thread."""
    import oracle
    from bit_groupwise_weight_amd.workloads import make_bias, make_weight, make_x
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        limit = threadpoolctl.threadpool_limits
    except Exception:
        threads, limit = 1, None
    model, nproc = host_cpu()
    prepared = []
    for c in cases:
        W = make_weight(c).numpy()
        ref = oracle.quantize(W, c.bits, c.group, c.act)
        x = make_x(c).float().numpy()
        b = make_bias(c)
        prepared.append((c, x, ref, None if b is None else b.float().numpy()))

    def run(n):
        nbytes, secs = 0, 0.0
        for c, x, ref, b in prepared:
            for _ in range(n):
                t0 = time.perf_counter()
                oracle.linear(x, ref["q"], ref["s"], ref["z"], c.group, b)
                secs += time.perf_counter() - t0
                nbytes += algo_bytes(c)
        return nbytes, secs

    total_bytes, total_s = run(reps)
    single = None
    if limit is not None:
        with limit(limits=1):
            b1, s1 = run(single_reps)
        single = {"value": round(b1 / s1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                  "sample": f"the same 7 cases, {single_reps} reps each, one BLAS thread, {s1:.1f} s"}
    return {"value": round(total_bytes / total_s / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"oracle linear (fp64 dequant + matmul) on the 7 decode cases "
                      f"K=N=4096 g64 bits 1..7, {reps} reps each, {total_s:.1f} s total; "
                      f"quantization excluded",
            "host": {"cpu_model": model, "nproc": nproc, "blas_threads": int(threads)},
            "single_thread": single}


# Workload configurations (bit_groupwise_weight_amd/workloads.py), by key.
CONFIG_GROUPS = [("single", "single decode", "single_qmv"),
                 ("llama8b", "Llama-3.1-8B decode", "llama8b_decode"),
                 ("llama_small", "Llama-3.2-1B/3B decode", "llama_small_decode"),
                 ("batched", "batched", "batched_qmm"),
                 ("mixed", "mixed sweep", "mixed_sweep")]
RIDGE_FLOP_PER_BYTE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)


def copies_for(c):
    return max(2, -(-ROTATE_BYTES // algo_bytes(c)))


def case_row(c, us):
    """Throughput of one case against its bounding roofline: HBM when the
    case's arithmetic intensity (2MNK flops per algorithmic byte) is below
    the ridge, MFMA above it."""
    nb, fl = algo_bytes(c), 2.0 * c.M * c.N * c.K
    gbps, tfs = nb / (us * 1e-6) / 1e9, fl / (us * 1e-6) / 1e12
    mfma = fl / nb > RIDGE_FLOP_PER_BYTE
    return {"case": c.name, "M": c.M, "K": c.K, "N": c.N, "bits": c.bits, "group": c.group,
            "act": c.act, "bias": c.bias, "us": round(us, 3), "bytes": nb,
            "GB_s": round(gbps, 1), "TFLOP_s": round(tfs, 2),
            "bound": "mfma" if mfma else "hbm",
            "frac": round(tfs / MFMA_BF16_PEAK_TFLOPS if mfma else gbps / HBM_PEAK_GBPS, 4)}


def all_configs(dev, stream, reps, only):
    """Every workload configuration, each case graph-timed over its own
    rotation of >= 1 GiB of weight copies; plus the single-launch floor (a
    plain read of the same bytes) at the wide Llama-3.1-8B decode shapes."""
    from bit_groupwise_weight_amd import workloads
    rows, summary, wide = [], [], []
    for key, label, fn in CONFIG_GROUPS:
        if only and key not in only:
            continue
        grows = []
        for c in getattr(workloads, fn)():
            p = prepare(c, copies_for(c), dev)
            torch.cuda.synchronize()
            n = len(p["sets"])
            g = capture(lambda i, s: launch(p, i, s), n, stream)
            us = time_graph(g, max(1, reps // n + 1), n, stream)
            del g, p
            torch.cuda.empty_cache()
            r = case_row(c, us)
            r["config"] = key
            grows.append(r)
            log(f"[{key}] {c.name}: {us:.3f} us  {r['GB_s']} GB/s  {r['TFLOP_s']} TFLOP/s  "
                f"({r['bound']} frac {r['frac']})")
            if key == "llama8b" and c.N != c.K and 1024 not in (c.N, c.K):
                wide.append((c, us))
        us_all = sorted(r["us"] for r in grows)
        summary.append({"config": key, "label": label, "cases": len(grows),
                        "us_min": us_all[0], "us_median": us_all[len(us_all) // 2],
                        "us_max": us_all[-1],
                        "frac_min": min(r["frac"] for r in grows),
                        "frac_median": sorted(r["frac"] for r in grows)[len(grows) // 2],
                        "frac_max": max(r["frac"] for r in grows)})
        rows += grows
    floor_wide = None
    if wide:
        reads = plain_read_us([algo_bytes(c) for c, _ in wide], dev, stream, reps)
        floor_wide = []
        for (c, us), (r_us, lpt) in zip(wide, reads):
            nb = algo_bytes(c)
            floor_wide.append({"case": c.name, "bytes": nb, "qmv_us": round(us, 3),
                               "stream_read_us": round(r_us, 3), "stream_read_loads_per_thread": lpt,
                               "stream_read_GB_s": round(nb / (r_us * 1e-6) / 1e9, 1),
                               "qmv_over_stream_read": round(us / r_us, 3),
                               "qmv_frac_hbm_peak": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
            log(f"floor {c.name}: plain read {r_us:.3f} us, qmv {us:.3f} us")
    return {"summary": summary, "cases": rows, "floor_wide": floor_wide,
            "note": "kernel us = HIP-event time of replays of a graph of back-to-back launches over "
                    "the case's own weight copies (>= 1 GiB) / launches; bound = mfma when "
                    "2MNK / algorithmic bytes exceeds the ridge (2.5 PFLOP/s / 8 TB/s), else hbm; "
                    "floor_wide = plain 16-byte streaming read of the same bytes in one launch"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path shards by output rows, see the design notes)", file=sys.stderr)
        sys.exit(2)
    from bit_groupwise_weight_amd import lowbit as lb
    lb.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 268435456 bytes read + 268435456 bytes written")

    qcases, mcases = qmv_cases(), qmm_cases()
    qmv_bytes_all = sum(algo_bytes(c) for c in qcases)
    qmm_bytes_all = sum(algo_bytes(c) for c in mcases)

    log("preparing: weight copies per case " +
        ", ".join(str(copies_for(c)) for c in qcases + mcases))
    qp = [prepare(c, copies_for(c), dev) for c in qcases]
    mp = [prepare(c, copies_for(c), dev) for c in mcases]
    torch.cuda.synchronize()

    def step(i, s):
        for p in qp:
            launch(p, i, s)
        for p in mp:
            launch(p, i, s)

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()

    # One graph per rotating copy index; each holds one full step.
    copies = min(len(p["sets"]) for p in qp + mp)
    step_graphs = [capture(lambda j, s, c=c: step(c, s), 1, stream) for c in range(copies)]
    torch.cuda.synchronize()
    for g in step_graphs:
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step_graphs[i % copies].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = e0.elapsed_time(e1) / args.steps
    log(f"timed {args.steps} steps (graph replay): {ms_per_step:.4f} ms/step "
        f"(host wall {wall_ms:.1f} ms)")

    # Per-kernel average launch durations: a graph of back-to-back launches
    # over all rotating copies, replayed; HIP events on the replay stream.
    def kernel_us(p):
        n = len(p["sets"])
        g = capture(lambda i, s: launch(p, i, s), n, stream)
        return time_graph(g, max(1, args.reps // n + 1), n, stream)

    qmv_us = [kernel_us(p) for p in qp]
    qmm_us = [kernel_us(p) for p in mp]
    eager_us = None if args.no_eager else [time_eager(p, args.reps, stream) for p in qp]
    eager_generic_us = None if args.no_eager else [time_eager(p, args.reps, stream, prepared=False)
                                                   for p in qp]
    per_bit = []
    for c, us in zip(qcases, qmv_us):
        gbps = algo_bytes(c) / (us * 1e-6) / 1e9
        per_bit.append({"bits": c.bits, "us": round(us, 3), "bytes": algo_bytes(c),
                        "GB_s": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)})
        log(f"qmv b={c.bits}: {us:.3f} us  {gbps:.1f} GB/s")
    qmv_total_us = sum(qmv_us)
    qmv_gbps = qmv_bytes_all / (qmv_total_us * 1e-6) / 1e9
    qmm = []
    for c, us in zip(mcases, qmm_us):
        fl = 2.0 * c.M * c.N * c.K
        tf = fl / (us * 1e-6) / 1e12
        qmm.append({"K": c.K, "N": c.N, "M": c.M, "us": round(us, 3), "TFLOP_s": round(tf, 2),
                    "frac_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        log(f"qmm K={c.K} N={c.N}: {us:.3f} us  {tf:.2f} TFLOP/s")
    # A decoder layer's linears (Llama-3.1-8B shapes, b=4, g=64, M=1): seven
    # separate launches vs four launches with the multi-linear entry point.
    lbytes = layer_bytes()
    decode_layer = None
    if not args.no_decode_layer:
        L = prepare_layer(max(2, -(-ROTATE_BYTES // lbytes)), dev)
        torch.cuda.synchronize()
        n = L["copies"]
        sep_us = time_graph(capture(lambda i, s: layer_separate(L, i, s), n, stream),
                            max(2, args.reps // n + 1), n, stream)
        fus_us = time_graph(capture(lambda i, s: layer_fused(L, i, s), n, stream),
                            max(2, args.reps // n + 1), n, stream)
        del L
        log(f"decoder layer linears: {sep_us:.2f} us as 7 launches, {fus_us:.2f} us as 4")
        decode_layer = {
            "model": "Llama-3.1-8B decoder layer linears (q,k,v,o,gate,up,down), M=1, bits 4, "
                     "group 64, fp16; synthetic weights; attention, norms and activations not "
                     "included",
            "bytes": lbytes,
            "separate_us": round(sep_us, 3), "separate_launches": 7,
            "fused_us": round(fus_us, 3), "fused_launches": 4,
            "fused_GB_s": round(lbytes / (fus_us * 1e-6) / 1e9, 1),
            "linear_only_us_per_token_32_layers": round(32 * fus_us, 2),
        }

    a8 = None if args.no_a8 else activation_quantized(dev, stream, args.reps)

    floor = None
    if not args.no_floor:
        floor = single_launch_floor([algo_bytes(c) for c in qcases], qmv_us, dev, stream, args.reps)

    fresh = kernel_source_hash() == MEASURED_TRAFFIC["src_hash"]
    qmv_traffic = MEASURED_TRAFFIC["qmv_bits1to7_bytes"] if fresh else None
    qmm_traffic = (sum(MEASURED_TRAFFIC["qmm_bytes"].values()) if fresh else None)
    qmm_util = MEASURED_TRAFFIC["qmm_mfma_util"] if fresh else None
    qmm_fl = sum(2.0 * c.M * c.N * c.K for c in mcases)
    qmm_tf = qmm_fl / (sum(qmm_us) * 1e-6) / 1e12

    out = {
        "metric": "qmv us & achieved HBM GB/s (bits 1-7, K=N=4096); qmm TFLOPS at M=128",
        "value": round(qmv_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,0.02) weights quantized on the GPU, N(0,1) activations)",
        "config": {
            "workload": "decode linears M=1 K=N=4096 group 64 fp16 bits 1..7 (qmv) + batched "
                        "M=128 bits 4 group 128 bf16 (K,N)=(4096,14336),(14336,4096) (qmm)",
            "rotating_weight_bytes": int(ROTATE_BYTES),
        },
        "roofline": {
            "kernel": "qmv (bits 1..7 instances, aggregated)",
            "bound": "hbm",
            "achieved": round(qmv_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(qmv_gbps / HBM_PEAK_GBPS, 4),
            "traffic": qmv_traffic,
            "traffic_note": "HBM bytes of one pass over the 7 launches (rocprofv3 FETCH_SIZE + "
                            "WRITE_SIZE, scaled); algorithmic bytes of that pass: "
                            + str(qmv_bytes_all),
        },
        "qmv_by_bits": per_bit,
        "single_launch_floor": floor,
        "qmv_total_us": round(qmv_total_us, 3),
        "roofline_qmm": {
            "kernel": "qmm (M=128, bits 4, group 128, bf16)",
            "bound": "mfma",
            "achieved": round(qmm_tf, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(qmm_tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": qmm_traffic,
            "traffic_note": "HBM bytes of the two shapes' launches incl. the split-K reduce "
                            "(rocprofv3, scaled); algorithmic bytes: " + str(qmm_bytes_all),
            "mfma_util_pct": qmm_util,
            "mfma_util_note": "rocprofv3 MfmaUtil of the main kernel per (K x N) shape, from the "
                              "profile of the same kernel sources; null for other sources",
        },
        "qmm": qmm,
        "activation_quantized": None if a8 is None else {
            "method": "8-bit dynamic activations (per-row symmetric int8, fp32 scale) x "
                      "groupwise low-bit weights on the int8 MFMA; M=128 bf16 x ~ N(0,1), "
                      "bits 4, group 32 (the -qmode 8da4w -G 32 export mode)",
            "cases": a8,
        },
        "roofline_a8": None if a8 is None else {
            "kernel": "qmm_a8 (int8 activations x 4-bit codes, group 32, M=128)",
            "bound": "mfma",
            "achieved": round(sum(2.0 * r["M"] * r["N"] * r["K"] for r in a8)
                              / (sum(r["linear_us"] for r in a8) * 1e-6) / 1e12, 2),
            "peak": MFMA_I8_PEAK_TOPS,
            "unit": "TOP/s",
            "frac": round(sum(2.0 * r["M"] * r["N"] * r["K"] for r in a8)
                          / (sum(r["linear_us"] for r in a8) * 1e-6) / 1e12 / MFMA_I8_PEAK_TOPS, 4),
            "traffic": (sum(MEASURED_TRAFFIC["a8_bytes"].get(f"{r['K']}x{r['N']}", 0) for r in a8)
                        if fresh and len(MEASURED_TRAFFIC["a8_bytes"]) == len(a8) else None),
            "traffic_note": "HBM bytes of one launch of each shape's linear (rocprofv3, scaled); "
                            "algorithmic bytes: codes + scales + zeros + int8 x + row scales + y",
        },
        "qmv_eager_us_per_call": None if eager_us is None else [round(u, 3) for u in eager_us],
        "qmv_eager_us_per_call_generic": None if eager_generic_us is None
        else [round(u, 3) for u in eager_generic_us],
        "decode_layer": decode_layer,
        "timing": "per-kernel us = HIP-event time of replays of a HIP graph of back-to-back "
                  "launches (rotating weight copies) / launches; steps replay one graph per "
                  "step; qmv_eager_us_per_call = one Python call per launch through a "
                  "PreparedLinear (weights validated once, output preallocated; host-bound); "
                  "_generic = through lowbit_linear, every tensor validated per call",
    }
    if args.all_configs:
        del qp, mp, step_graphs
        torch.cuda.empty_cache()
        only = set(k for k in args.only_configs.split(",") if k)
        out["all_configs"] = all_configs(dev, stream, args.reps, only)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline(qcases, args.cpu_sample_reps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
