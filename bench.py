#!/usr/bin/env python3
"""Throughput of wav2vec2-CTC encoder inference on one MI355X.

One step = one pass of the whole path over one batch: w2v2_forward_greedy
(conv feature encoder, feature projection, positional conv, transformer
blocks, CTC head with the per-frame argmax in its epilogue, greedy CTC
collapse), inputs already resident in device memory.  Default workload:
wav2vec2-base shape, 16 s windows (256000 samples, 799 frames), batch 8,
fp16 operands with fp32 accumulation and normalisation, seeded random
weights and seeded speech-like synthetic PCM with valid lengths 2-16 s.

Prints one JSON line:
  value        audio-seconds per second (RTFx): batch * window seconds / step
               time, from the K timed steps (HIP events on the stream)
  pages_method median of 7 interleaved rounds x K steps, eager and replayed
               from a captured HIP graph (the timing method of the TensorRT
               wav2vec2 README, "Method")
  stages       frontend / encoder time from event pairs at the stage boundary
               inside the concurrent (product) execution
  sweep        the base 16 s x 32 workload: throughput and stage split
  roofline     the dominant kernel's achieved rate against the MI355X peak,
               from its algorithmic work per launch and its average launch
               duration measured with HIP events (one-stream roofline pass)
  cpu_baseline the CPU oracle (float64 numpy) on a bounded sample of the same
               workload, on this host's cores; cpu_baseline_per_config: the
               oracle in float64 and float32 on one row of every workload
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "audio-sec/sec (RTFx) + ms/window, wav2vec2-base 16 s batch 8, 1 MI355X"
PEAK_FP16_TFLOPS = 2500.0     # MI355X dense fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
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
        # conv 1.. outputs: normalised in place (read and write the operand type)
        w["conv_ln_gelu"] = ("byte", sum(2.0 * dsize * B * T[i] * C[i] for i in range(1, len(C))))
    w["gemm_feature_proj"] = ("flop", 2.0 * M * d * C[-1])
    w["pos_conv_gemm"] = ("flop", 2.0 * M * d * K * (d // G))
    w["gemm_qkv"] = ("flop", L * 2.0 * M * 3 * d * d)
    w["gemm_out_proj"] = ("flop", L * 2.0 * M * d * d)
    w["gemm_ffn1"] = ("flop", L * 2.0 * M * F * d)
    w["gemm_ffn2"] = ("flop", L * 2.0 * M * d * F)
    w["gemm_ctc_head"] = ("flop", 2.0 * M * cfg.vocab * d)
    w["attention"] = ("flop", L * 4.0 * B * H * Tf * Tf * (d // H))
    # LayerNorms: the encoder's read the fp32 residual and write the operand
    # copy (post-norm: plus (mean, rstd) per row); the feature projection's
    # reads the last conv output and writes the operand copy.
    n_ln = 2 * L + 1
    per_ln = M * d * (4.0 + dsize) + (0.0 if cfg.stable_layer_norm else 8.0 * M)
    w["layernorm"] = ("byte", n_ln * per_ln + M * C[-1] * 2.0 * dsize)
    w["pos_pack"] = ("byte", M * d * 4.0 + G * B * (Tf + K) * (d // G) * dsize)
    return w


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(blas) if blas else 1
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(cfg, W, pcm, valid, rows: int, dtype_name: str = "float64") -> dict:
    """The oracle, unchanged, on the first `rows` rows of the batch."""
    import numpy as np

    import oracle
    sub = cfg.replace(batch=rows)
    dt = np.float64 if dtype_name == "float64" else np.float32
    t0 = time.perf_counter()
    logits, vf = oracle.forward(sub, W, pcm[:rows], valid[:rows], dtype=dt)
    oracle.greedy_decode(logits, vf, cfg.blank_id)
    dt_s = time.perf_counter() - t0
    audio = rows * cfg.window / 16000.0
    return {"value": round(audio / dt_s, 3), "unit": "audio-sec/sec", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"{rows} of {cfg.batch} rows of {cfg.name} ({audio:.0f} s of padded window audio), "
                      f"{dtype_name} numpy oracle incl. argmax+collapse, {dt_s:.1f} s wall",
            "host_cpus": len(os.sched_getaffinity(0)), "seconds": round(dt_s, 2),
            "frames_check": int(np.sum(vf))}


def read_traffic(kernel: str, workload: str, precision: str,
                 key: str = "traffic_bytes_per_launch") -> float | None:
    """HBM bytes per launch of `kernel` (its full-batch launches of the
    roofline pass) from a committed rocprofv3 counter summary, if one exists
    for this workload, precision and the current kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    # the kernel's sources: every file listed, hashed in order
    h = hashlib.sha256()
    for name in kv.get("source", "").split():
        src = os.path.join(ROOT, "wav2vec2_ctc_encoder_amd", "csrc", name)
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    if h.hexdigest()[:16] != kv.get("source_sha16"):
        return None
    if kv.get("workload") != workload or kv.get("precision") != precision:
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


class Workload:
    """One model with its seeded inputs and output buffers on cuda:0."""

    def __init__(self, cfg, dev, W=None, precision=None):
        import torch

        import synth
        import wav2vec2_ctc_encoder_amd as w2
        self.cfg = cfg
        self.W = synth.make_weights(cfg) if W is None else W
        self.pcm, self.valid = synth.make_pcm(cfg)
        self.model = w2.Model(cfg, self.W, device=0, precision=precision)
        B, T = cfg.batch, self.model.frames_per_window
        self.T = T
        self.tp = torch.from_numpy(self.pcm).to(dev)
        self.tv = torch.from_numpy(self.valid).to(dev)
        self.logits = torch.empty(B, T, cfg.vocab, dtype=torch.float32, device=dev)
        self.vf = torch.empty(B, dtype=torch.int32, device=dev)
        self.ids = torch.empty(B, T, dtype=torch.int32, device=dev)
        self.lens = torch.empty(B, dtype=torch.int32, device=dev)

    def step(self):
        self.model.forward_greedy(self.tp, self.tv, self.logits, self.vf, self.ids, self.lens)

    @property
    def audio_s(self) -> float:
        return self.cfg.batch * self.cfg.window / 16000.0

    def timed(self, steps: int, fn=None) -> float:
        """ms per step over `steps` calls of fn, bracketed by synchronizations
        and one event pair on the current stream."""
        import torch
        fn = fn or self.step
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def stages(self, steps: int) -> dict:
        """Per-part frontend / encoder time from the library's stage event
        pairs, in the unchanged concurrent execution."""
        self.model.profile_enable(True, "stage")
        for _ in range(steps):
            self.step()
        import torch
        torch.cuda.synchronize()
        r = self.model.profile_read()
        self.model.profile_enable(False)
        out = {}
        for k in ("stage_frontend", "stage_encoder"):
            if k in r:
                ms, n = r[k]
                out[k.replace("stage_", "") + "_ms"] = round(ms / n, 4)
                out["parts_per_step"] = n // steps
        return out

    def pages_method(self, steps: int, rounds: int, graph: bool) -> dict:
        """Median of `rounds` rounds of `steps` steps, eager and (if capture
        works) replayed from one captured HIP graph, the rounds interleaved."""
        import torch
        res = {"rounds": rounds, "steps_per_round": steps}
        g = None
        if graph:
            try:
                ref_logits = self.logits.clone()
                ref_ids = self.ids.clone()
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(s):
                    self.step()          # a warm call on the capture stream
                torch.cuda.current_stream().wait_stream(s)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    self.step()
                torch.cuda.synchronize()
                self.logits.zero_()
                self.ids.zero_()
                g.replay()
                torch.cuda.synchronize()
                res["graph_matches_eager"] = bool(torch.equal(self.logits, ref_logits) and
                                                  torch.equal(self.ids, ref_ids))
            except Exception as e:  # capture unsupported: report eager only
                res["graph_error"] = f"{type(e).__name__}: {e}"[:300]
                g = None
        eager, replay = [], []
        for _ in range(rounds):
            eager.append(self.timed(steps))
            if g is not None:
                replay.append(self.timed(steps, g.replay))
        res["eager"] = {"median_ms": round(statistics.median(eager), 4),
                        "rounds_ms": [round(x, 4) for x in eager]}
        if replay:
            res["graph"] = {"median_ms": round(statistics.median(replay), 4),
                            "rounds_ms": [round(x, 4) for x in replay]}
        for k in ("eager", "graph"):
            if k in res:
                ms = res[k]["median_ms"]
                res[k]["audio_sec_per_sec"] = round(self.audio_s / (ms / 1e3), 1)
                res[k]["ms_per_window"] = round(ms / self.cfg.batch, 4)
        return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="base_16s_b8")
    ap.add_argument("--precision", default=None, help="fp16 (default of the workload) or fp32")
    ap.add_argument("--rounds", type=int, default=7, help="interleaved rounds of the pages' timing method (0: skip)")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay rounds")
    ap.add_argument("--sweep", default="base_16s_b32", help="second workload timed beside the first ('none': skip)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-projection leg")
    ap.add_argument("--cpu-rows", type=int, default=2, help="rows the CPU oracle baseline runs (0: skip)")
    ap.add_argument("--cpu-configs", default="all", help="'all': one-row oracle baselines of every workload; 'none'")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a device copy of this many MiB (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not implemented (windows are independent, "
              "so a multi-GPU run would split the batch across GPUs with no communication)", file=sys.stderr)
        return 2

    import torch

    import synth

    cfg = synth.PRESETS[args.workload]
    if args.precision:
        cfg = cfg.replace(precision=args.precision)
    B = cfg.batch
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wl = Workload(cfg, dev)
    model, T = wl.model, wl.T
    print(f"[bench] workload {cfg.name} B={B} window={cfg.window} frames={T} precision={cfg.precision}",
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        wl.step()
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

    def roofline(kernel, ms_total, launches, steps):
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
        r["traffic"] = read_traffic(kernel, cfg.name, cfg.precision)
        r["kernel"] = kernel
        r["avg_launch_ms"] = round(avg_s * 1e3, 4)
        r["launches_per_step"] = launches / steps
        r["work_per_launch"] = per_launch
        r["work_unit"] = kind
        return r

    # Timed region (right after the warmup): K steps of the product path (the
    # batch halves run concurrently on two streams), bracketed by
    # synchronizations and two events and nothing else.
    t_wall0 = time.perf_counter()
    ms_step = wl.timed(args.steps)
    t_wall = time.perf_counter() - t_wall0
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)
    window_s = cfg.window / 16000.0
    value = B * window_s / (ms_step / 1e3)
    valid_s = float(wl.valid.sum()) / 16000.0

    # Roofline pass: K steps with events around every kernel.  With every
    # kernel profiled the library runs the whole batch as one pass on one
    # stream, so each launch runs alone and its event-timed duration is the
    # kernel's own (it agrees with the profiler's kernel trace).  This pass
    # gives the per-kernel table, the dominant kernel and its roofline.
    model.profile_enable(True)
    ms_serial = wl.timed(args.steps)
    per_kernel = model.profile_read()
    model.profile_enable(False)
    dominant = max(per_kernel, key=lambda k: per_kernel[k][0])
    roof = roofline(dominant, per_kernel[dominant][0], per_kernel[dominant][1], args.steps)
    roof["pass"] = ("roofline pass: the same workload, K steps with events around every launch; the batch runs "
                    "as one pass on one stream so each launch runs alone")
    print(f"[bench] roofline pass done ({ms_serial:.3f} ms/step); dominant kernel {dominant}", file=sys.stderr,
          flush=True)

    pages = wl.pages_method(args.steps, args.rounds, not args.no_graph) if args.rounds > 0 else None
    if pages:
        print(f"[bench] pages' method: eager median {pages['eager']['median_ms']:.3f} ms"
              + (f", graph median {pages['graph']['median_ms']:.3f} ms" if "graph" in pages else ""),
              file=sys.stderr, flush=True)
    stages = wl.stages(args.steps)

    # true-length leg: the same rows, each computed as its own clip of its
    # valid[b] samples (rows packed, work proportional to the valid audio);
    # reported beside the padded-window metric, never as `value`
    import wav2vec2_ctc_encoder_amd as w2
    tl_logits = torch.empty_like(wl.logits)

    def tl_step():
        model.forward_true_length(wl.tp, wl.valid, tl_logits, wl.vf)
        w2.ctc_greedy(tl_logits, wl.vf, cfg.blank_id, wl.ids, wl.lens)

    for _ in range(args.warmup):
        tl_step()
    tl_ms = wl.timed(args.steps, tl_step)
    print(f"[bench] true-length mode: {tl_ms:.3f} ms/step", file=sys.stderr, flush=True)

    kernels = {}
    for k, (ms, n) in sorted(per_kernel.items(), key=lambda kv: -kv[1][0]):
        ent = {"ms_per_step": round(ms / args.steps, 4), "launches_per_step": n // args.steps}
        if k in work:
            kk, amt = work[k]
            rate = amt / (ms / args.steps / 1e3)
            if kk == "flop":
                ent["tflops"] = round(rate / 1e12, 1)
                ent["frac_of_peak"] = round(rate / 1e12 / (PEAK_FP16_TFLOPS if dsize == 2 else PEAK_FP32_TFLOPS), 4)
            else:
                ent["gbs"] = round(rate / 1e9, 1)
                ent["frac_of_peak"] = round(rate / 1e9 / PEAK_HBM_GBS, 4)
            # HBM-side bytes from the committed counter summary (fp16 kernels of this workload)
            tr = read_traffic(k, cfg.name, cfg.precision)
            if tr is not None:
                ent["traffic_bytes_per_launch"] = tr
                ent["traffic_gbs"] = round(tr / (ms / n / 1e3) / 1e9, 1)
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
                   else "fp32", "valid_audio_s": round(valid_s, 2),
                   "step": "w2v2_forward_greedy: forward + per-frame argmax in the CTC head + collapse"},
        "rtfx_valid_audio": round(valid_s / (ms_step / 1e3), 1),
        "pages_method": pages,
        "stages": dict(stages, mode="two concurrent halves (product path); per-half event pairs at the "
                                    "frontend / encoder boundary"),
        "true_length": {"ms_per_step": round(tl_ms, 4), "valid_audio_sec_per_sec": round(valid_s / (tl_ms / 1e3), 1),
                        "speedup_over_padded": round(ms_step / tl_ms, 3),
                        "mode": "each row computed as its own clip of valid[b] samples, rows packed"},
        "wall_s_timed": round(t_wall, 3),
        "stages_ms_roofline_pass": {"frontend": round(fe, 4), "encoder_head_ctc": round(enc, 4)},
        "kernels": kernels,
        "roofline": roof,
        "ms_per_step_roofline_pass": round(ms_serial, 4),
    }
    W, pcm, valid = wl.W, wl.pcm, wl.valid

    # fp8 leg: the same workload with the q/k/v/out/fc1/fc2 projections on
    # e4m3 operands (TensorRT README, "FP8 quantization study"), calibrated
    # by the library itself on windows of another PCM seed
    if not args.no_fp8 and cfg.precision == "fp16" and cfg.hidden % 128 == 0 and cfg.ffn % 128 == 0:
        cal_pcm, cal_valid = synth.make_pcm(cfg, seed=cfg.pcm_seed + 50)
        amax = model.calibrate(torch.from_numpy(cal_pcm).to(dev), torch.from_numpy(cal_valid).to(dev))
        torch.cuda.synchronize()
        w8 = Workload(cfg, dev, W=dict(W, **w2.amax_table(amax)), precision="fp8")
        for _ in range(args.warmup):
            w8.step()
        ms8 = w8.timed(args.steps)
        w8.model.profile_enable(True)
        w8.timed(args.steps)
        pk8 = w8.model.profile_read()
        w8.model.profile_enable(False)
        fp8 = {"precision": "fp8 e4m3 projections (per-tensor scales, static activation calibration), "
                            "fp16 graph otherwise",
               "calibration": f"w2v2_calibrate of the fp16 model on {cfg.batch} windows of PCM seed "
                              f"{cfg.pcm_seed + 50}",
               "ms_per_step": round(ms8, 4), "audio_sec_per_sec": round(wl.audio_s / (ms8 / 1e3), 1),
               "speedup_over_fp16": round(ms_step / ms8, 3)}
        if args.rounds > 0:
            fp8["pages_method_eager"] = w8.pages_method(args.steps, args.rounds, graph=False)["eager"]
            if pages:
                fp8["speedup_over_fp16_medians"] = round(pages["eager"]["median_ms"] /
                                                         fp8["pages_method_eager"]["median_ms"], 3)
        gk = {}
        for k in ("gemm_qkv", "gemm_out_proj", "gemm_ffn1", "gemm_ffn2"):
            if k in pk8 and k in work:
                ms, n = pk8[k]
                rate = work[k][1] / (ms / args.steps / 1e3) / 1e12
                gk[k] = {"ms_per_step": round(ms / args.steps, 4), "tflops": round(rate, 1),
                         "frac_of_fp8_peak": round(rate / PEAK_FP8_TFLOPS, 4),
                         "fp16_ms_per_step": kernels.get(k, {}).get("ms_per_step")}
        fp8["gemms_roofline_pass"] = gk
        print(f"[bench] fp8 projections: {ms8:.3f} ms/step ({ms_step / ms8:.3f}x)", file=sys.stderr, flush=True)
        out["fp8"] = fp8
        w8.model.close()
        del w8

    model.close()
    del wl
    torch.cuda.empty_cache()

    if args.sweep and args.sweep != "none":
        scfg = synth.PRESETS[args.sweep]
        sw = Workload(scfg, dev)
        for _ in range(args.warmup):
            sw.step()
        sms = sw.timed(args.steps)
        s_valid = float(sw.valid.sum()) / 16000.0
        sweep = {"workload": scfg.name, "batch": scfg.batch, "ms_per_step": round(sms, 4),
                 "ms_per_window": round(sms / scfg.batch, 4),
                 "audio_sec_per_sec": round(sw.audio_s / (sms / 1e3), 1),
                 "rtfx_valid_audio": round(s_valid / (sms / 1e3), 1),
                 "stages": sw.stages(args.steps)}
        if args.rounds > 0:
            pm = sw.pages_method(args.steps, args.rounds, graph=False)
            sweep["pages_method_eager"] = pm["eager"]
        print(f"[bench] sweep {scfg.name}: {sms:.3f} ms/step", file=sys.stderr, flush=True)
        out["sweep"] = sweep
        sw.model.close()
        del sw
        torch.cuda.empty_cache()

    if args.cpu_rows > 0:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, W, pcm, valid, min(args.cpu_rows, B))
    else:
        out["cpu_baseline"] = None
    if args.cpu_configs == "all":
        per = {}
        for name, pc in synth.PRESETS.items():
            pW = synth.make_weights(pc)
            ppcm, pvalid = synth.make_pcm(pc)
            per[name] = {dn: cpu_baseline(pc, pW, ppcm, pvalid, 1, dn) for dn in ("float64", "float32")}
            print(f"[bench] cpu baseline {name}: " + ", ".join(
                f"{dn} {v['value']} audio-s/s" for dn, v in per[name].items()), file=sys.stderr, flush=True)
        out["cpu_baseline_per_config"] = per
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
