#!/usr/bin/env python3
"""Throughput of wav2vec2-CTC encoder inference on one MI355X.

One step = one pass of the whole path over one batch: w2v2_forward (conv
feature encoder, feature projection, positional conv, transformer blocks,
CTC head) + w2v2_ctc_greedy (per-frame argmax and collapse), inputs already
resident in device memory.  Default workload: wav2vec2-base shape, 16 s
windows (256000 samples, 799 frames), batch 8, fp16 operands with fp32
accumulation and normalisation, seeded random weights and seeded
speech-like synthetic PCM with valid lengths 2-16 s.

Prints one JSON line:
  value        audio-seconds per second (RTFx): batch * window seconds / step time
  ms_per_step  mean step time over the K timed steps (HIP events on the stream)
  roofline     the dominant kernel's achieved rate against the MI355X peak,
               from its algorithmic work per launch and its average launch
               duration measured with HIP events inside the timed region
  cpu_baseline the CPU oracle (float64 numpy) on a bounded sample of the same
               workload, on this host's cores
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

METRIC = "audio-sec/sec (RTFx) + ms/window, wav2vec2-base 16 s batch 8, 1 MI355X"
PEAK_FP16_TFLOPS = 2500.0     # MI355X dense fp16 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

FRONTEND_KERNELS = {"gn0_stats", "gn0_finalize", "conv0_gn_gelu", "conv0_ln_gelu", "conv_ln_gelu"} | \
    {f"conv{i}_gemm" for i in range(1, 8)}


def frames(n, ks, ss):
    out = []
    for k, s in zip(ks, ss):
        n = 0 if n < k else (n - k) // s + 1
        out.append(n)
    return out


def algorithmic_work(cfg, B: int, dsize: int) -> dict[str, tuple[str, float]]:
    """Algorithmic work per step for each kernel name: ("flop" | "byte", amount).

    Contractions count 2*M*N*K flops; memory-bound kernels count the bytes
    they must read and write once (inputs, outputs and fp32 statistics).
    """
    T = frames(cfg.window, cfg.conv_kernel, cfg.conv_stride)
    Tf = T[-1]
    C = cfg.conv_dim
    d, F, H, G, K = cfg.hidden, cfg.ffn, cfg.heads, cfg.pos_groups, cfg.pos_kernel
    M = B * Tf
    L = cfg.layers
    w = {}
    for i in range(1, len(C)):
        w[f"conv{i}_gemm"] = ("flop", 2.0 * B * T[i] * C[i] * cfg.conv_kernel[i] * C[i - 1])
    if cfg.feat_norm == "group":
        # conv0 + GroupNorm + GELU: read the PCM, write the normalised output once
        w["conv0_gn_gelu"] = ("byte", B * cfg.window * 4.0 + B * T[0] * C[0] * dsize)
        w["gn0_stats"] = ("byte", B * cfg.window * 4.0)
    else:
        w["conv0_ln_gelu"] = ("byte", B * cfg.window * 4.0 + B * T[0] * C[0] * dsize)
        w["conv_ln_gelu"] = ("byte", sum(2.0 * B * T[i] * C[i] * dsize for i in range(1, len(C))))
    w["gemm_feature_proj"] = ("flop", 2.0 * M * d * C[-1])
    w["pos_conv_gemm"] = ("flop", 2.0 * M * d * K * (d // G))
    w["gemm_qkv"] = ("flop", L * 2.0 * M * 3 * d * d)
    w["gemm_out_proj"] = ("flop", L * 2.0 * M * d * d)
    w["gemm_ffn1"] = ("flop", L * 2.0 * M * F * d)
    w["gemm_ffn2"] = ("flop", L * 2.0 * M * d * F)
    w["gemm_ctc_head"] = ("flop", 2.0 * M * cfg.vocab * d)
    w["attention"] = ("flop", L * 4.0 * B * H * Tf * Tf * (d // H))
    # LayerNorms of the encoder: read the fp32 residual, write the operand copy
    # (+ the fp32 residual again in the post-norm layout), plus the feature LN.
    n_ln = 2 * L + 1
    per_ln = M * d * (4.0 + dsize + (0.0 if cfg.stable_layer_norm else 4.0))
    w["layernorm"] = ("byte", n_ln * per_ln + M * C[-1] * 2.0 * dsize)
    w["pos_pack"] = ("byte", M * d * 4.0 + G * B * (Tf + K) * (d // G) * dsize)
    return w


def cpu_baseline(cfg, W, pcm, valid, rows: int) -> dict:
    """The oracle, unchanged, on the first `rows` rows of the batch."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max(blas) if blas else 1
    except Exception:  # pragma: no cover
        threads = 1
    sub = cfg.replace(batch=rows)
    t0 = time.perf_counter()
    logits, vf = oracle.forward(sub, W, pcm[:rows], valid[:rows])
    oracle.greedy_decode(logits, vf, cfg.blank_id)
    dt = time.perf_counter() - t0
    audio = rows * cfg.window / 16000.0
    return {"value": round(audio / dt, 3), "unit": "audio-sec/sec", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} of {cfg.batch} rows of {cfg.name} ({audio:.0f} s of padded window audio), "
                      f"float64 numpy oracle incl. argmax+collapse, {dt:.1f} s wall",
            "host_cpus": len(os.sched_getaffinity(0)), "seconds": round(dt, 2),
            "frames_check": int(np.sum(vf))}


def read_traffic(kernel: str, key: str = "traffic_bytes_per_launch") -> float | None:
    """HBM bytes per launch of `kernel` (its one-pass launches of the
    roofline pass) from a committed rocprofv3 counter summary, if one exists
    for the current kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    # the kernel's sources: every file listed (the GEMM and the header whose
    # device functions it inlines), hashed in order
    h = hashlib.sha256()
    for name in kv.get("source", "").split():
        src = os.path.join(ROOT, "wav2vec2_ctc_encoder_amd", "csrc", name)
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    sha = h.hexdigest()[:16]
    if sha != kv.get("source_sha16"):
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="base_16s_b8")
    ap.add_argument("--precision", default=None, help="fp16 (default of the workload) or fp32")
    ap.add_argument("--cpu-rows", type=int, default=2, help="rows the CPU oracle baseline runs (0: skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a device copy of this many MiB (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not implemented (windows are independent, "
              "so a multi-GPU run would split the batch across GPUs with no communication)", file=sys.stderr)
        return 2

    import torch

    import synth
    import wav2vec2_ctc_encoder_amd as w2

    cfg = synth.PRESETS[args.workload]
    if args.precision:
        cfg = cfg.replace(precision=args.precision)
    B = cfg.batch
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    model = w2.Model(cfg, W, device=0)
    tp = torch.from_numpy(pcm).to(dev)
    tv = torch.from_numpy(valid).to(dev)
    T = model.frames_per_window
    logits = torch.empty(B, T, cfg.vocab, dtype=torch.float32, device=dev)
    vf = torch.empty(B, dtype=torch.int32, device=dev)
    ids = torch.empty(B, T, dtype=torch.int32, device=dev)
    lens = torch.empty(B, dtype=torch.int32, device=dev)

    def step():
        model.forward(tp, tv, logits, vf)
        w2.ctc_greedy(logits, vf, cfg.blank_id, ids, lens)

    print(f"[bench] workload {cfg.name} B={B} window={cfg.window} frames={T} precision={cfg.precision}",
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    dsize = 2 if cfg.precision == "fp16" else 4
    work = algorithmic_work(cfg, B, dsize)

    def roofline(kernel, ms_total, launches, steps, traffic_key):
        """Algorithmic work per launch of `kernel` over its event-timed
        average launch duration."""
        kind, amount = work.get(kernel, ("flop", float("nan")))
        per_launch = amount / (launches / steps)
        avg_s = ms_total / launches / 1e3
        if kind == "flop":
            achieved = per_launch / avg_s / 1e12
            peak = PEAK_FP16_TFLOPS if cfg.precision == "fp16" else PEAK_FP32_TFLOPS
            r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s"}
        else:
            achieved = per_launch / avg_s / 1e9
            r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        r["frac"] = round(achieved / r["peak"], 4)
        r["traffic"] = read_traffic(kernel, traffic_key)
        r["kernel"] = kernel
        r["avg_launch_ms"] = round(avg_s * 1e3, 4)
        r["launches_per_step"] = launches / steps
        r["work_per_launch"] = per_launch
        r["work_unit"] = kind
        return r

    # Roofline pass: K steps with events around every kernel.  With every
    # kernel profiled the library runs the whole batch as one pass on one
    # stream, so each launch runs alone and its event-timed duration is the
    # kernel's own (it agrees with the profiler's kernel trace).  This pass
    # gives the per-kernel table, the dominant kernel and its roofline.
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    model.profile_enable(True)
    prof_steps = args.steps
    ev0.record(stream)
    for _ in range(prof_steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_serial = ev0.elapsed_time(ev1) / prof_steps
    per_kernel = model.profile_read()
    model.profile_enable(False)
    dominant = max(per_kernel, key=lambda k: per_kernel[k][0])
    roof = roofline(dominant, per_kernel[dominant][0], per_kernel[dominant][1], prof_steps,
                    "traffic_bytes_per_launch")
    roof["pass"] = ("roofline pass: the same workload, K steps with events around every launch; the batch runs "
                    "as one pass on one stream so each launch runs alone")
    print(f"[bench] roofline pass done ({ms_serial:.3f} ms/step); dominant kernel {dominant}", file=sys.stderr,
          flush=True)

    # Timed region: K steps of the product path (the batch halves run
    # concurrently on two streams), bracketed by two events and nothing else.
    # Per-kernel events are not used here: with two streams an event pair
    # around a launch also spans the time the kernel waits for CUs that the
    # other half's kernels hold.
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)

    window_s = cfg.window / 16000.0
    value = B * window_s / (ms_step / 1e3)
    valid_s = float(valid.sum()) / 16000.0

    # true-length leg: the same rows, each computed as its own clip of its
    # valid[b] samples (rows packed, work proportional to the valid audio);
    # reported beside the padded-window metric, never as `value`
    tl_logits = torch.empty_like(logits)

    def tl_step():
        model.forward_true_length(tp, valid, tl_logits, vf)
        w2.ctc_greedy(tl_logits, vf, cfg.blank_id, ids, lens)

    for _ in range(args.warmup):
        tl_step()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        tl_step()
    ev1.record(stream)
    torch.cuda.synchronize()
    tl_ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] true-length mode: {tl_ms:.3f} ms/step", file=sys.stderr, flush=True)

    kernels = {}
    for k, (ms, n) in sorted(per_kernel.items(), key=lambda kv: -kv[1][0]):
        ent = {"ms_per_step": round(ms / prof_steps, 4), "launches_per_step": n // prof_steps}
        if k in work:
            kk, amt = work[k]
            rate = amt / (ms / prof_steps / 1e3)
            if kk == "flop":
                ent["tflops"] = round(rate / 1e12, 1)
            else:
                ent["gbs"] = round(rate / 1e9, 1)
        kernels[k] = ent
    fe = sum(v["ms_per_step"] for k, v in kernels.items() if k in FRONTEND_KERNELS)
    enc = sum(v["ms_per_step"] for k, v in kernels.items() if k not in FRONTEND_KERNELS)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "audio-sec/sec", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_window": round(ms_step / B, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.precision, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "window_s": window_s, "frames": T,
                   "precision": "fp16 operands, fp32 accumulation/normalisation" if cfg.precision == "fp16"
                   else "fp32", "valid_audio_s": round(valid_s, 2)},
        "rtfx_valid_audio": round(valid_s / (ms_step / 1e3), 1),
        "true_length": {"ms_per_step": round(tl_ms, 4), "valid_audio_sec_per_sec": round(valid_s / (tl_ms / 1e3), 1),
                        "speedup_over_padded": round(ms_step / tl_ms, 3),
                        "mode": "each row computed as its own clip of valid[b] samples, rows packed"},
        "wall_s_timed": round(t_wall, 3),
        "stages_ms": {"frontend": round(fe, 4), "encoder_head_ctc": round(enc, 4)},
        "kernels": kernels,
        "roofline": roof,
        "ms_per_step_roofline_pass": round(ms_serial, 4),
    }
    model.close()
    if args.cpu_rows > 0:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, W, pcm, valid, min(args.cpu_rows, B))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
