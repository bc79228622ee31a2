"""Throughput of the Matryoshka multi-exit hot path on one MI355X.

One step = both junctions (block 1 -> 2, block 2 -> 3), the rewrite of the
three row-major heads into the MFMA-tiled layout, every exit's head, the
distillation loss and dL/dlogits for all three exits, on one batch of seeded
synthetic inputs shaped like the 500M / 1.5B / 3B suite (widths 1024, 2304,
4352; vocabulary 32768; 8 x 2048 tokens; bf16 inputs, fp32 accumulation;
alpha_d = 0.3).  Inputs are resident in HBM before timing.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints one JSON line.  Per-kernel durations come from HIP events that the
library records around every launch on the launch stream during the timed
steps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
WORKLOAD = 2


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Sources that make up the head GEMM whose HBM traffic the counter runs measured.
GEMM_SOURCES = ("heads_packed.hip", "wave128_core.h", "packed16_core.h", "packed_core.h", "common.h",
                "tiles.h", "internal.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nested_exit_lm_amd", "csrc")
    for f in GEMM_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(p=None):
    """HBM bytes per launch of the head GEMM from rocprofv3 counter runs, if they
    were taken on the current kernel sources (else None).  p: the record
    (default profiles/traffic.json)."""
    p = p or os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("heads_loss_bytes_per_launch")


def _blas_info():
    """BLAS library NumPy calls (vendor, version, threads), via threadpoolctl."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"vendor": i.get("internal_api"), "version": i.get("version"),
                        "threads": int(i.get("num_threads", 1))}
    except Exception:
        pass
    return {"vendor": None, "version": None, "threads": os.cpu_count()}


def _oracle_rate(oracle, s, seconds, chunk=256):
    """Tokens/s of the oracle's forward (junctions, heads, losses, dlogits) on
    the first tokens of the batch, `chunk` at a time, until `seconds` pass."""
    done = 0
    t0 = time.perf_counter()
    while done < s.n_tokens:
        rows = np.arange(done, min(done + chunk, s.n_tokens))
        for m in range(1, s.n_exits):
            oracle.junction(s.h[m - 1][rows], s.ids[rows], s.emb[m])
        oracle.forward_tokens(s.h, s.w, s.labels, s.alpha, 1.0, rows=rows, chunk=chunk)
        done += len(rows)
        if time.perf_counter() - t0 > seconds:
            break
    return done, time.perf_counter() - t0


def cpu_baseline(s, seconds: float):
    """The oracle, as it stands, on a bounded sample of the same workload: the
    first tokens of the batch, 256 at a time, until `seconds` have passed; in
    float64 (the parity oracle: `value`) and again in float32 (the same
    definitions in single precision: `value_fp32`)."""
    import oracle
    blas = _blas_info()
    done, el = _oracle_rate(oracle, s, seconds)
    with oracle.working_precision(np.float32):
        done32, el32 = _oracle_rate(oracle, s, seconds / 2)
    return {"value": done / el, "unit": "tokens/s", "cores": blas["threads"], "kind": "oracle",
            "value_fp32": done32 / el32, "host_cpus": os.cpu_count(), "blas": blas,
            "sample": f"first {done} of {s.n_tokens} tokens of the same batch (NumPy oracle: "
                      f"{s.n_exits - 1} junctions, {s.n_exits} heads, losses and dlogits) in float64, "
                      f"{el:.1f} s; first {done32} tokens in float32, {el32:.1f} s; "
                      f"{blas['threads']} BLAS threads ({blas['vendor']} {blas['version']}) "
                      f"on {os.cpu_count()} host CPUs"}


def junction_cold(nel, torch, dev, hs, ids, embs, j2, j3, jbytes, s, reps=10):
    """Both junctions timed with a cold last-level cache: before each pair a
    512 MiB buffer is overwritten, which evicts the 256 MB MALL, so the first
    read of every embedding row comes from HBM.  Repeated rows of the Zipf ids
    within one launch may still hit in the caches; `distinct_row_bytes` is the
    traffic if every distinct embedding row were read exactly once."""
    evict = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ms = []
    for _ in range(reps):
        evict.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        nel.junction(hs[0], ids, embs[1], out=j2)
        nel.junction(hs[1], ids, embs[2], out=j3)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b) / 2)
    ms.sort()
    med = ms[len(ms) // 2]
    D, N = s.widths, s.n_tokens
    nd = len(np.unique(s.ids))
    distinct = sum(2 * (D[m - 1] * N + (D[m] - D[m - 1]) * nd + D[m] * N) + 4 * N for m in (1, 2)) / 2
    del evict
    return {"cold_avg_ms": med, "cold_gbs": jbytes / 2 / (med / 1e3) / 1e9,
            "cold_hbm_frac": jbytes / 2 / (med / 1e3) / 1e9 / HBM_PEAK_GBS,
            "distinct_ids": nd, "distinct_row_bytes": distinct,
            "cold_gbs_distinct_rows": distinct / (med / 1e3) / 1e9}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-verify", action="store_true", help="skip the speculative-verify sub-benchmark")
    ap.add_argument("--no-backward", action="store_true", help="skip the head-backward sub-benchmark")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the sub-benchmark of the divergences and junction modes")
    ap.add_argument("--no-reference", "--no-probe", dest="no_reference", action="store_true",
                    help="skip the reference measurement: the vendor library's plain GEMM on "
                         "the widest exit's shape (--no-probe is the older name)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB read + 1 GiB write kernel three times (the "
                         "reference that scales the HBM byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line: one JSON line with the loss step of "
                         "every training-shaped workload (tiny f32, 200M proxy, 500M/1.5B/3B, "
                         "4 exits), the verify shape, and a bounded oracle sample for each")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="read the rocprofv3 FETCH_SIZE / WRITE_SIZE runs, write "
                         "profiles/traffic.json, and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path is built and timed on a single MI355X "
              "(token sharding across GPUs is described, not built). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import nested_exit_lm_amd as nel

    nel.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep:
        print(json.dumps({"sweep": bench_sweep(nel, torch, synth, dev, args)}), flush=True)
        return
    log("[bench] generating inputs")
    s = synth.make_workload(WORKLOAD)
    N, V, D = s.n_tokens, s.vocab, s.widths

    def td(a):
        return torch.from_numpy(synth.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)

    hs = [td(x) for x in s.h]
    ws = [td(x) for x in s.w]
    embs = [td(x) for x in s.emb]
    ids = torch.from_numpy(s.ids).to(dev)
    labels = torch.from_numpy(s.labels).to(dev)
    j2 = torch.empty(N, D[1], dtype=torch.bfloat16, device=dev)
    j3 = torch.empty(N, D[2], dtype=torch.bfloat16, device=dev)
    pw = [torch.empty_like(w) for w in ws]
    dl = [torch.empty(N, V, dtype=torch.bfloat16, device=dev) for _ in D]
    mean = torch.empty(3 * len(D) + 1, dtype=torch.float32, device=dev)
    tok = torch.empty(len(D), 3, N, dtype=torch.float32, device=dev)
    wsb = torch.zeros(nel.workspace_size(nel.OP_LOSS, len(D), N, V), dtype=torch.uint8, device=dev)

    def step():
        nel.junction(hs[0], ids, embs[1], out=j2)
        nel.junction(hs[1], ids, embs[2], out=j3)
        for w, p in zip(ws, pw):
            nel.pack_weights(w, out=p)
        nel.matryoshka_loss_packed(hs, pw, labels, alpha_d=s.alpha, grad_scale=1.0, dlogits=dl,
                                   workspace=wsb, mean_loss=mean, token_loss=tok)

    if args.calibrate_copy:
        log("[bench] copy calibration: 3 x (read 1 GiB, write 1 GiB)")
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del a, b
    log("[bench] warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nel.timing_reset()
    nel.timing_enable(True)
    log(f"[bench] timing {args.steps} steps")
    # events on the stream every kernel is launched on, around each step
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    nel.timing_enable(False)
    ms = (t1 - t0) * 1e3 / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    kern = {}
    for k in ("junction", "pack", "heads_loss", "merge", "means", "finalize"):
        tot, cnt = nel.timing_read(k)
        kern[k] = {"avg_ms": tot / max(cnt, 1), "launches": cnt}

    flops = 2.0 * N * V * sum(D)                                   # head GEMM, per launch
    k2 = kern["heads_loss"]["avg_ms"] / 1e3
    jbytes = sum(2 * (D[m - 1] + (D[m] - D[m - 1]) + D[m]) * N + 4 * N for m in (1, 2))  # both junctions
    fbytes = 2 * len(D) * N * V * 2                               # finalize: read s, write g
    pbytes = 2 * V * sum(D) * 2 / len(D)                          # pack: read + write, per launch
    kern["heads_loss"]["tflops"] = flops / k2 / 1e12
    kern["heads_loss"]["mfma_frac"] = flops / k2 / 1e12 / BF16_PEAK_TFLOPS
    kern["junction"]["gbs"] = jbytes / 2 / (kern["junction"]["avg_ms"] / 1e3) / 1e9
    kern["junction"]["hbm_frac"] = kern["junction"]["gbs"] / HBM_PEAK_GBS
    kern["finalize"]["gbs"] = fbytes / (kern["finalize"]["avg_ms"] / 1e3) / 1e9
    kern["finalize"]["hbm_frac"] = kern["finalize"]["gbs"] / HBM_PEAK_GBS
    kern["pack"]["gbs"] = pbytes / (kern["pack"]["avg_ms"] / 1e3) / 1e9
    kern["pack"]["hbm_frac"] = kern["pack"]["gbs"] / HBM_PEAK_GBS
    # merge: read (m, sigma) per (exit, statistics tile, token), the label logits and
    # labels; write LSE and (CE, Dist, L) per (exit, token).  The statistics tiles
    # are 128 entries wide from the one-wavefront-per-SIMD loss GEMM (mean exit
    # width of at least 512) and 256 from the two-workgroups-per-CU one.
    tile = 128 if sum(D) >= 512 * len(D) else 256
    n_vt = (V + tile - 1) // tile
    mbytes = 4 * N * (2 * len(D) * n_vt + len(D) + 1 + len(D) + 3 * len(D))
    kern["merge"]["gbs"] = mbytes / (kern["merge"]["avg_ms"] / 1e3) / 1e9
    kern["merge"]["hbm_frac"] = kern["merge"]["gbs"] / HBM_PEAK_GBS
    kern["junction"].update(junction_cold(nel, torch, dev, hs, ids, embs, j2, j3, jbytes, s))
    traffic = measured_traffic()
    losses = mean.cpu().numpy().tolist()
    out = {
        "metric": "tokens/s of junction+3-exit head+distill loss (fwd+dlogits)",
        "value": N / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": per_step[len(per_step) // 2],
        "ms_per_step_min": per_step[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": s.name, "widths": list(D), "vocab": V, "batch": s.batch,
                   "seq_len": s.seq, "tokens": N, "alpha_d": s.alpha, "exits": len(D),
                   "accumulate": "fp32", "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "kernel": "heads_loss", "achieved": flops / k2 / 1e12,
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / k2 / 1e12 / BF16_PEAK_TFLOPS, "traffic": traffic},
        "kernels": kern,
        "end_to_end_mfma_frac": flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
        "mean_loss": losses,
    }
    if not args.no_reference:
        out["reference"] = bench_reference(torch, dev)
    if not args.no_verify:
        out["verify_102x7"] = bench_verify(nel, torch, synth, dev, args)
    if not args.no_backward:
        out["backward"] = bench_backward(nel, torch, hs, ws, dl, args, ids=ids, embs=embs,
                                         pw=pw, labels=labels, alpha=s.alpha)
    if not args.no_variants:
        out["variants"] = bench_variants(nel, torch, hs, pw, labels, dl, wsb, mean, tok, s.alpha,
                                         args, ids=ids, embs=embs)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline")
        out["cpu_baseline"] = cpu_baseline(s, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def _read_counter_csv(d):
    """{kernel name: [counter value per dispatch]} from a rocprofv3 --pmc run directory."""
    import csv
    import glob
    out = {}
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def summarize_counters(fetch_dir, write_dir, out=None):
    """HBM traffic per launch of the head GEMM: rocprofv3 FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled so that the calibration kernel (1 GiB read,
    1 GiB written) reads exactly its size.  Written to `out` (default
    profiles/traffic.json) and returned."""
    fetch, write = _read_counter_csv(fetch_dir), _read_counter_csv(write_dir)

    def pick(dct, key):
        names = [k for k in dct if key in k]
        if not names:
            raise KeyError(f"no kernel matching {key}")
        vals = [v for k in names for v in dct[k]]
        return names[0], vals

    gib_kib = float(1 << 20)
    _, cf = pick(fetch, "AUnaryFunctor")     # the calibration kernel: b = a * 1.0 over 1 GiB
    _, cw = pick(write, "AUnaryFunctor")
    f_scale = gib_kib / (sorted(cf)[len(cf) // 2])
    w_scale = gib_kib / (sorted(cw)[len(cw) // 2])
    name, hf = pick(fetch, "heads_loss_kernel<3>")
    _, hw = pick(write, "heads_loss_kernel<3>")
    fb = sum(hf) / len(hf) * 1024 * f_scale
    wb = sum(hw) / len(hw) * 1024 * w_scale
    res = {"source_hash": kernel_source_hash(), "kernel": name,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "heads_loss_fetch_bytes": fb, "heads_loss_write_bytes": wb,
           "heads_loss_bytes_per_launch": fb + wb}
    out = out or os.path.join(ROOT, "profiles", "traffic.json")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))
    return res


def bench_backward(nel, torch, hs, ws, dl, args, ids=None, embs=None, pw=None, labels=None,
                   alpha=0.3):
    """Backward of the three exit heads on the step's own logit gradients:
    dh_m = G_m W^m (bf16) and dW^m = G_m^T h_m (fp32), with the W and h operand packs;
    the backward of both junctions on seeded synthetic upstream gradients; and (with
    the packed heads and labels) the loss plus head backward with stored gradients
    against the fused call that never stores them."""
    N, V = dl[0].shape
    D = [h.shape[1] for h in hs]
    need = nel.heads_backward_workspace_size(N, V, D)
    wsb = torch.empty(need, dtype=torch.uint8, device=hs[0].device)
    dhs = [torch.empty_like(h) for h in hs]
    dws = [torch.empty(V, d, dtype=torch.float32, device=h.device) for h, d in zip(hs, D)]
    steps = max(args.steps // 2, 3)

    def per_exit():
        for m in range(len(D)):
            nel.head_backward(dl[m], hs[m], ws[m], dh=dhs[m], dw=dws[m], workspace=wsb)

    def step():   # one grouped dh launch and one grouped dW launch for all exits
        nel.heads_backward(dl, hs, ws, dhs=dhs, dws=dws, workspace=wsb)

    per_exit()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        per_exit()
    torch.cuda.synchronize()
    per_exit_ms = (time.perf_counter() - t0) * 1e3 / steps
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    nel.timing_reset()
    nel.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    nel.timing_enable(False)
    res = {"ms_per_step": (t1 - t0) * 1e3 / steps,
           "per_exit_calls_ms_per_step": per_exit_ms,
           "work": "dh (bf16) and dW (fp32) of all three heads from the step's dlogits"}
    flops = 2.0 * N * V * sum(D)          # per GEMM kind, all exits
    for k in ("bwd_pack", "bwd_dh", "bwd_dw"):
        tot, cnt = nel.timing_read(k)
        res[k + "_ms"] = tot / steps
    res["dh_tflops"] = flops / (res["bwd_dh_ms"] / 1e3) / 1e12
    res["dw_tflops"] = flops / (res["bwd_dw_ms"] / 1e3) / 1e12
    res["dh_mfma_frac"] = res["dh_tflops"] / BF16_PEAK_TFLOPS
    res["dw_mfma_frac"] = res["dw_tflops"] / BF16_PEAK_TFLOPS
    if ids is not None:
        g = torch.Generator(device=hs[0].device)
        g.manual_seed(7)
        douts = [(torch.randn(N, D[m], generator=g, device=hs[0].device) * 1e-2).bfloat16()
                 for m in (1, 2)]
        jdh = [torch.empty_like(hs[m]) for m in (0, 1)]
        jde = [torch.empty(V, D[m] - D[m - 1], dtype=torch.float32, device=hs[0].device)
               for m in (1, 2)]

        def jstep():
            for i, m in enumerate((1, 2)):
                nel.junction_backward(hs[m - 1], ids, embs[m], douts[i], dh=jdh[i], demb=jde[i])

        jstep()
        torch.cuda.synchronize()
        nel.timing_reset()
        nel.timing_enable(True)
        for _ in range(steps):
            jstep()
        torch.cuda.synchronize()
        nel.timing_enable(False)
        tot, cnt = nel.timing_read("junction_bwd")
        # per token: read h, dout, the embedding row; write dh; per vocabulary row: write demb
        jbytes = sum(N * (2 * D[m - 1] + 2 * D[m] + 2 * (D[m] - D[m - 1]) + 2 * D[m - 1] + 4)
                     + V * 4 * (D[m] - D[m - 1]) for m in (1, 2))
        res["junction_bwd_ms"] = tot / steps
        res["junction_bwd_gbs"] = jbytes / (tot / steps / 1e3) / 1e9
    if pw is not None and labels is not None:
        res["fused"] = bench_fused(nel, torch, hs, ws, pw, labels, dl, dhs, dws, wsb, alpha, steps)
    return res


def bench_fused(nel, torch, hs, ws, pw, labels, dl, dhs, dws, bwd_ws, alpha, steps):
    """Loss plus the backward of every head, two ways on the same inputs: stored
    (the loss writes the logit gradients G, then the grouped dh and dW GEMMs read
    them) and fused (one call; the dh and dW GEMMs form G from the loss pass's fp16
    scratch, bit-identical results, G never written).  The dl buffers serve as the
    stored gradients and as the fused call's scratch."""
    N, V = dl[0].shape
    D = [h.shape[1] for h in hs]
    M = len(D)
    dev = hs[0].device
    lw = torch.zeros(nel.workspace_size(nel.OP_LOSS, M, N, V), dtype=torch.uint8, device=dev)
    fw = torch.zeros(nel.loss_backward_workspace_size(N, V, D), dtype=torch.uint8, device=dev)
    mean = torch.empty(3 * M + 1, dtype=torch.float32, device=dev)
    tok = torch.empty(M, 3, N, dtype=torch.float32, device=dev)

    def stored():
        nel.matryoshka_loss_packed(hs, pw, labels, alpha_d=alpha, dlogits=dl, workspace=lw,
                                   mean_loss=mean, token_loss=tok)
        nel.heads_backward(dl, hs, ws, dhs=dhs, dws=dws, workspace=bwd_ws)

    def fused():
        nel.loss_backward_packed(hs, ws, pw, labels, alpha_d=alpha, scratch=dl, dhs=dhs,
                                 dws=dws, mean_loss=mean, token_loss=tok, workspace=fw)

    flops = 2.0 * N * V * sum(D)          # per GEMM kind (forward, dh, dW), all exits
    out = {"work": "loss (fwd + gradients) and dh, dW of all three heads; the weight "
                   "packs (W^T, h^T) included, the forward's weight pack not",
           "steps": steps}
    names = ("heads_loss", "merge", "finalize", "means", "grad_consts", "bwd_pack", "bwd_dh",
             "bwd_dw")
    for key, fn in (("stored", stored), ("fused", fused)):
        fn()
        torch.cuda.synchronize()
        nel.timing_reset()
        nel.timing_enable(True)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        nel.timing_enable(False)
        k = {}
        for nm in names:
            tot, cnt = nel.timing_read(nm)
            if cnt:
                k[nm + "_ms"] = tot / steps
        k["dh_tflops"] = flops / (k["bwd_dh_ms"] / 1e3) / 1e12
        k["dw_tflops"] = flops / (k["bwd_dw_ms"] / 1e3) / 1e12
        k["dh_mfma_frac"] = k["dh_tflops"] / BF16_PEAK_TFLOPS
        k["dw_mfma_frac"] = k["dw_tflops"] / BF16_PEAK_TFLOPS
        out[key] = {"ms_per_step": e0.elapsed_time(e1) / steps,
                    "tokens_per_s": N / (e0.elapsed_time(e1) / steps / 1e3), "kernels": k}
    out["fused_speedup"] = out["stored"]["ms_per_step"] / out["fused"]["ms_per_step"]
    del lw, fw
    return out


def bench_reference(torch, dev):
    """Context, not part of the path: the vendor library's plain GEMM
    (torch.matmul, hipBLASLt) on the widest exit's head shape, with the
    benchmark's operand distributions and no epilogue."""
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    N, V, D = 16384, 32768, 4352
    h = (torch.randn(N, D, generator=g, device=dev) * 4.0).bfloat16()
    w = (torch.randn(V, D, generator=g, device=dev) * 0.02).bfloat16()
    torch.matmul(h, w.t())
    times = []
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            torch.matmul(h, w.t())
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / 5)
    ms = sorted(times)[1]
    tf = 2.0 * N * V * D / (ms / 1e3) / 1e12
    del h, w
    return {"vendor_gemm": {"what": "torch.matmul (hipBLASLt), h [16384, 4352] x W^T "
                                    "[4352, 32768] bf16, fp32 accumulation, bf16 output",
                            "tflops": tf, "frac_of_peak": tf / BF16_PEAK_TFLOPS}}


def bench_variants(nel, torch, hs, pw, labels, dl, wsb, mean, tok, alpha, args, ids, embs):
    """The same loss step (packed heads, already packed) with each other
    divergence and with per-exit weights, and junction 2 -> 3 in each mode.
    The divergence pass reads the stored shifted logits of every exit once."""
    N, V = dl[0].shape
    D = [h.shape[1] for h in hs]
    M = len(D)
    steps = max(args.steps // 4, 3)

    def timed(fn, kernel):
        fn()
        torch.cuda.synchronize()
        nel.timing_reset()
        nel.timing_enable(True)
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        nel.timing_enable(False)
        tot, _ = nel.timing_read(kernel)
        return (t1 - t0) * 1e3 / steps, tot / steps

    res = {"steps": steps, "work": "packed heads + loss + dlogits (no junction, no weight packing)"}
    for name, div, lam in (("forward", 0, None), ("forward_weighted", 0, [0.5, 1.0, 2.0]),
                           ("reverse_kl", 1, None), ("js", 2, None), ("tv", 3, None)):
        ms, dms = timed(lambda: nel.matryoshka_loss_packed(
            hs, pw, labels, alpha_d=alpha, dlogits=dl, workspace=wsb, mean_loss=mean,
            token_loss=tok, exit_weights=lam, divergence=div), "divergence")
        r = {"ms_per_step": ms}
        if div:
            r["divergence_pass_ms"] = dms
            r["divergence_pass_gbs"] = M * N * V * 2 / (dms / 1e3) / 1e9   # reads every exit's s
        res[name] = r
    out = torch.empty(N, D[2], dtype=hs[0].dtype, device=hs[0].device)
    for name, mode in (("rescale", 0), ("no_rescale", 1), ("zero_fill", 2)):
        ms, jms = timed(lambda: nel.junction(hs[1], ids, embs[2], out=out, mode=mode), "junction")
        res["junction_2to3_" + name + "_ms"] = jms
    return res


def bench_sweep(nel, torch, synth, dev, args):
    """The loss step (every junction, the weight packs, heads + loss + dlogits) of
    workloads 0-3, timed like the benchmark line, with the per-kernel rates and a
    bounded oracle sample; then the verify shape."""
    res = []
    for k in range(4):
        s = synth.make_workload(k)
        log(f"[sweep] workload {k} ({s.name})")
        N, V, D, M = s.n_tokens, s.vocab, s.widths, s.n_exits
        f32 = s.dtype == "f32"
        es = 4 if f32 else 2

        def td(a):
            if f32:
                return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
            return torch.from_numpy(synth.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)

        hs = [td(x) for x in s.h]
        ws = [td(x) for x in s.w]
        embs = [td(x) for x in s.emb]
        ids = torch.from_numpy(s.ids).to(dev)
        labels = torch.from_numpy(s.labels).to(dev)
        js = [torch.empty(N, D[m], dtype=hs[0].dtype, device=dev) for m in range(1, M)]
        pw = None if f32 else [torch.empty_like(w) for w in ws]
        dl = [torch.empty(N, V, dtype=hs[0].dtype, device=dev) for _ in D]
        mean = torch.empty(3 * M + 1, dtype=torch.float32, device=dev)
        tok = torch.empty(M, 3, N, dtype=torch.float32, device=dev)
        wsb = torch.zeros(nel.workspace_size(nel.OP_LOSS, M, N, V), dtype=torch.uint8, device=dev)

        def step():
            for m in range(1, M):
                nel.junction(hs[m - 1], ids, embs[m], out=js[m - 1])
            if f32:
                nel.matryoshka_loss(hs, ws, labels, alpha_d=s.alpha, dlogits=dl, workspace=wsb,
                                    mean_loss=mean, token_loss=tok)
            else:
                for w, p in zip(ws, pw):
                    nel.pack_weights(w, out=p)
                nel.matryoshka_loss_packed(hs, pw, labels, alpha_d=s.alpha, dlogits=dl,
                                           workspace=wsb, mean_loss=mean, token_loss=tok)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        nel.timing_reset()
        nel.timing_enable(True)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        nel.timing_enable(False)

        def avg(kname):
            tot, cnt = nel.timing_read(kname)
            return tot / max(cnt, 1)

        jms, kms, fms = avg("junction"), avg("heads_loss"), avg("finalize")
        jbytes = sum(es * (D[m - 1] + (D[m] - D[m - 1]) + D[m]) * N + 4 * N
                     for m in range(1, M)) / (M - 1)                     # per junction launch
        fbytes = 2 * M * N * V * es
        flops = 2.0 * N * V * sum(D)
        row = {"workload": s.name, "tokens": N, "widths": list(D), "vocab": V, "dtype": s.dtype,
               "ms_per_step": ms, "tokens_per_s": N / (ms / 1e3),
               "junction_ms": jms, "junction_gbs": jbytes / (jms / 1e3) / 1e9,
               "heads_loss_ms": kms, "heads_loss_tflops": flops / (kms / 1e3) / 1e12,
               "finalize_ms": fms, "finalize_gbs": fbytes / (fms / 1e3) / 1e9,
               "merge_ms": avg("merge")}
        row["junction_hbm_frac"] = row["junction_gbs"] / HBM_PEAK_GBS
        row["heads_loss_mfma_frac"] = row["heads_loss_tflops"] / BF16_PEAK_TFLOPS
        row["finalize_hbm_frac"] = row["finalize_gbs"] / HBM_PEAK_GBS
        if not args.no_cpu_baseline:
            row["cpu_baseline"] = cpu_baseline(s, args.cpu_seconds / 3)
        res.append(row)
        del hs, ws, embs, js, pw, dl, wsb
        torch.cuda.empty_cache()
    if not args.no_verify:
        log("[sweep] verify shape")
        v = bench_verify(nel, torch, synth, dev, args)
        v["workload"] = "spec-verify-102x7"
        res.append(v)
    return res


def bench_verify(nel, torch, synth, dev, args):
    """Speculative-verify shape: junction 1 -> 2, heads of exits 1 and 3 with greedy
    argmax, accepted prefix length (102 sequences x 7 positions)."""
    s = synth.make_workload(4)

    def td(a):
        return torch.from_numpy(synth.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)

    hs = [td(s.h[m]) for m in s.exits]
    # decoding reuses the same heads every step: they are packed once, up front
    ws = [nel.pack_weights(td(s.w[m])) for m in s.exits]
    emb = td(s.emb[1])
    ids = torch.from_numpy(s.ids).to(dev)
    j = torch.empty(s.n_tokens, s.widths[1], dtype=torch.bfloat16, device=dev)
    wsb = torch.zeros(nel.workspace_size(nel.OP_HEADS, 2, s.n_tokens, s.vocab), dtype=torch.uint8,
                      device=dev)

    def step():
        nel.junction(hs[0], ids, emb, out=j)
        _, am = nel.exit_heads_packed(hs, ws, want_logits=False, want_argmax=True, workspace=wsb)
        nel.accept_prefix(am[0].view(s.batch, s.seq), am[1].view(s.batch, s.seq), 6)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nel.timing_reset()
    nel.timing_enable(True)
    steps = max(args.steps, 20)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    nel.timing_enable(False)
    tot, cnt = nel.timing_read("heads_argmax")
    flops = 2.0 * s.n_tokens * s.vocab * (s.widths[0] + s.widths[2])
    k = tot / max(cnt, 1) / 1e3
    # sampled verification (nucleus 0.9, T = 1): heads with fp32 logits, then
    # acceptance and the next-token draw from uniforms drawn up front
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    B, P = s.batch, s.seq
    toks = torch.randint(0, s.vocab, (B, P), generator=g, device=dev, dtype=torch.int32)
    ua = torch.rand(B, P, generator=g, device=dev)
    un = torch.rand(B, generator=g, device=dev)

    def sstep():
        nel.junction(hs[0], ids, emb, out=j)
        lg, _ = nel.exit_heads_packed(hs, ws, want_logits=True, want_argmax=False, workspace=wsb)
        nel.speculative_verify(lg[0], lg[1], toks, ua, un, 6, temperature=1.0, top_p=0.9)

    for _ in range(args.warmup):
        sstep()
    torch.cuda.synchronize()
    nel.timing_reset()
    nel.timing_enable(True)
    t2 = time.perf_counter()
    for _ in range(steps):
        sstep()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    nel.timing_enable(False)
    stot, _ = nel.timing_read("speculative")
    return {"ms_per_step": (t1 - t0) * 1e3 / steps, "tokens": s.n_tokens,
            "sampled_ms_per_step": (t3 - t2) * 1e3 / steps,
            "speculative_kernels_ms": stot / steps,
            "weights": "packed once before timing (static heads in decoding)",
            "heads_argmax_ms": k * 1e3, "heads_argmax_tflops": flops / k / 1e12,
            "heads_argmax_mfma_frac": flops / k / 1e12 / BF16_PEAK_TFLOPS}


if __name__ == "__main__":
    main()
