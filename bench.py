#!/usr/bin/env python3
"""KDA on one MI355X: prefill tokens/s at H=32, d=128, T=64K and decode state
GB/s, each against its roofline, with the fp64 oracle timed on the host.

One step = the whole hot path over one batch of synthetic input:
  prefill  kda_chunk_prep + kda_chunk_state_pass (= kda_chunk_fwd) over
           B=1, T=65536, H=32, dk=dv=128, bf16 inputs, fp32 state and output
  decode   64 kda_decode_step launches over N=256 requests x H=32 heads with
           resident fp32 states (128x128), bf16 per-token inputs
Inputs are generated on the GPU before timing (seeded, synthetic). Every
kernel launch is bracketed by HIP events on the stream it runs on.

After the timed steps: the options built on the path (bf16 output,
snapshots, speculative verify/commit, the span-by-span prefill through the
context-split entry points), the other forward workloads, and the fp64 C
oracle (test infrastructure) on the host's cores beside every workload,
whose outputs also check the GPU's element by element.

Prints one JSON line. `value` is prefill tokens/s (B*T / prefill time).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H=32,d=128,T=64K) + decode state GB/s, % of roofline"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
FP32_MFMA_PEAK_TFLOPS = 157.3   # dense fp32 matrix
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
PREFILL_MFMA_TARGET = 0.40      # stated target for the prefill, as a fraction of bf16 peak
DECODE_HBM_TARGET = 0.70        # stated target for the decode step, as a fraction of HBM peak


def log(*parts):
    print("[bench]", *parts, file=sys.stderr, flush=True)


def prefill_units(dk, dv, in_bytes=2, C=16):
    """Algorithmic work per token-head of the prefill path (fp32 o):
    flops 6 dk dv + 4C dk + 2C dv + C(dk+dv); bytes q,k,g,v + beta in, o out."""
    flops = 6 * dk * dv + 4 * C * dk + 2 * C * dv + C * (dk + dv)
    bytes_ = in_bytes * (3 * dk + dv + 1) + 4 * dv
    return flops, bytes_


class ClockSampler:
    """The shader clock during the timed steps, as the driver reports it: the
    current level of pp_dpm_sclk (the line marked '*'), read from sysfs every
    few milliseconds by a background thread. Reads a file only; never touches
    the GPU. None where the file is missing or unreadable."""

    PERIOD_S = 0.005

    def __init__(self):
        import glob
        self.path = next((p for p in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
                          if os.access(p, os.R_OK)), None)
        self.samples = []
        self._stop = None
        self._thread = None

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def start(self):
        if self.path is None:
            return
        import threading
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                mhz = self._read()
                if mhz is not None:
                    self.samples.append(mhz)
                self._stop.wait(self.PERIOD_S)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is None:
            return None
        self._stop.set()
        self._thread.join()
        if not self.samples:
            return None
        xs = sorted(self.samples)
        return {"source": self.path.replace("/device/pp_dpm_sclk", "") + " pp_dpm_sclk (current level)",
                "samples": len(xs), "min_mhz": xs[0], "median_mhz": xs[len(xs) // 2],
                "max_mhz": xs[-1], "peak_mhz": 2400}


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(kernel):
    """HBM traffic per dispatch measured with rocprofv3 counters, if it was
    taken on the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = rec.get("kernels", {}).get(kernel)
    if not ent or ent.get("source_sha256") != source_sha(ent.get("sources", [])):
        return None
    return ent.get("bytes_per_dispatch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg")
    ap.add_argument("--cpu-1m-tokens", type=int, default=16384,
                    help="leading tokens (all heads) of the 1M-token workload the oracle runs")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the option measurements and the other forward workloads "
                         "(profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested). Run with --gpus 1." % args.gpus, file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_attention_recurrence_11_amd import binding, configs, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pf = configs.PREFILL_64K
    dc = configs.DECODE
    B, T, H, dk, dv = pf.B, pf.T, pf.H, pf.dk, pf.dv
    log("generating %s and %s" % (pf.name, dc.name))
    ins = inputs.make_workload(pf, device=dev)
    code = 1  # bf16 inputs
    ws = torch.empty(binding.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, code),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    ST = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    d = inputs.make_workload(dc, device=dev)
    N, steps = dc.B, dc.T
    # one untimed 64-step run from the workload's initial states, kept for the
    # oracle's check; the timed steps then advance a copy in place
    S0_dec = d["S"].clone()
    S = d["S"].clone()
    dec_check = [binding.kda_decode_step(d["q"][s], d["k"][s], d["v"][s], d["g"][s], d["beta"][s], S)
                 for s in range(steps)]
    dec_check = (torch.stack(dec_check).cpu(), S.cpu())
    S.copy_(S0_dec)
    o_dec = torch.empty((N, dc.H, dc.dv), dtype=torch.float32, device=dev)
    copy_src = copy_dst = None
    if args.copy_calibration:
        copy_src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)   # 1 GiB
        copy_dst = torch.empty_like(copy_src)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def step(evs):
        e = evs
        e[0].record(stream)
        binding.kda_chunk_prep(ins["q"], ins["k"], ins["g"], ins["beta"], dv, workspace=ws)
        e[1].record(stream)
        binding.kda_chunk_state_pass(ins["v"], ws, dk, ins["S0"], o=o, S_T=ST)
        e[2].record(stream)
        for s in range(steps):
            e[3 + 2 * s].record(stream)
            binding.kda_decode_step(d["q"][s], d["k"][s], d["v"][s], d["g"][s], d["beta"][s], S, o=o_dec)
            e[4 + 2 * s].record(stream)
        if copy_src is not None:
            copy_dst.copy_(copy_src)

    nev = 3 + 2 * steps
    new_events = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step(new_events())
    torch.cuda.synchronize()

    log("timing %d steps" % args.steps)
    all_ev = [new_events() for _ in range(args.steps)]
    clock = ClockSampler()
    torch.cuda.synchronize()
    clock.start()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(all_ev[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gpu_clock = clock.stop()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    prep_ms = np.array([e[0].elapsed_time(e[1]) for e in all_ev])
    pass_ms = np.array([e[1].elapsed_time(e[2]) for e in all_ev])
    dec_ms = np.array([[e[3 + 2 * s].elapsed_time(e[4 + 2 * s]) for s in range(steps)] for e in all_ev])
    prefill_ms = prep_ms + pass_ms
    # host copies for the oracle's check of this workload (o of the last step)
    pf_check = (o.cpu(), ST.cpu())

    nxt = None
    if not args.no_next:
        nxt = measure_next(binding, inputs, ins, ws, o, ST, d, B, T, H, dk, dv, stream, dev, np,
                           torch)
    tokens = B * T
    value = tokens / (prefill_ms.mean() * 1e-3)

    # ---- rooflines (algorithmic work / measured average launch time) ----
    th = B * T * H
    f_tok, b_tok = prefill_units(dk, dv)
    state_bytes = 2 * dk * dv * 4                         # state read + write
    prep_bytes = th * (2 * 3 * dk + 2)                    # q, k, g, beta in
    pass_bytes = th * (2 * dv + 4 * dv) + B * H * dk * dv * 4  # v in, o out, S_T out (S0 = 0)
    path_bytes = th * b_tok + B * H * dk * dv * 4
    dec_unit_bytes = state_bytes + 2 * (3 * dc.dk + dc.dv) + 2 + 4 * dc.dv
    dec_bytes = N * dc.H * dec_unit_bytes
    dec_state_bytes = N * dc.H * state_bytes

    def roof(name, nbytes, ms, bound="hbm"):
        achieved = nbytes / (ms * 1e-3) / 1e9
        return {"kernel": name, "bound": bound, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic(name), "algorithmic_bytes_per_launch": int(nbytes),
                "avg_launch_us": round(ms * 1e3, 2)}

    r_dec = roof("kda_decode_kernel", dec_bytes, dec_ms.mean())
    r_dec["target_frac"] = DECODE_HBM_TARGET
    r_prep = roof("kda_chunk_prep", prep_bytes, prep_ms.mean())
    r_pass = roof("kda_state_pass", pass_bytes, pass_ms.mean())
    step_share = {"kda_decode_kernel": dec_ms.sum(1).mean(), "kda_chunk_prep": prep_ms.mean(),
                  "kda_state_pass": pass_ms.mean()}
    dominant = max(step_share, key=step_share.get)
    roofs = {"kda_decode_kernel": r_dec, "kda_chunk_prep": r_prep, "kda_state_pass": r_pass}
    prefill_gbps = path_bytes / (prefill_ms.mean() * 1e-3) / 1e9
    prefill_tflops = th * f_tok / (prefill_ms.mean() * 1e-3) / 1e12
    # the prefill path's own roofline, beside the headline value it belongs to:
    # HBM-bound at this shape (74.6 flop/B < the ~315 flop/B ridge), reported
    # against both peaks; the matrix-core fraction counts algorithmic flops only
    roof_prefill = {
        "path": "kda_chunk_prep + kda_chunk_state_pass", "bound": "hbm",
        "achieved": round(prefill_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(prefill_gbps / HBM_PEAK_GBPS, 4),
        "traffic": (None if load_traffic("kda_chunk_prep") is None or load_traffic("kda_state_pass") is None
                    else load_traffic("kda_chunk_prep") + load_traffic("kda_state_pass")),
        "algorithmic_bytes_per_launch": int(path_bytes), "avg_ms": round(prefill_ms.mean(), 4),
        "mfma_achieved_TFLOPs": round(prefill_tflops, 2), "mfma_peak_TFLOPs": BF16_MFMA_PEAK_TFLOPS,
        "mfma_frac": round(prefill_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "mfma_target_frac": PREFILL_MFMA_TARGET,
        "mfma_frac_at_hbm_roof": round(f_tok / b_tok / (BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)), 4),
    }

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": pf.name, "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "chunk": 16,
                   "in_dtype": "bf16", "state_dtype": "f32", "out_dtype": "f32",
                   "decode_workload": dc.name, "decode_requests": N, "decode_steps": steps},
        "roofline": roofs[dominant],
        "roofline_prefill": roof_prefill,
        "gpu_clock_during_timed_steps": gpu_clock,
        "roofline_decode": r_dec,
        "prefill": {
            "tokens_per_s": round(value, 1), "ms": round(prefill_ms.mean(), 4),
            "median_ms": round(float(np.median(prefill_ms)), 4),
            "prep_ms": round(prep_ms.mean(), 4), "state_pass_ms": round(pass_ms.mean(), 4),
            "algorithmic_GBps": round(prefill_gbps, 1),
            "frac_of_hbm_roof": round(prefill_gbps / HBM_PEAK_GBPS, 4),
            "algorithmic_TFLOPs": round(prefill_tflops, 2),
            "frac_of_bf16_mfma_peak": round(prefill_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "bytes_per_token_head": b_tok, "flops_per_token_head": f_tok,
        },
        "decode": {
            "state_GBps": round(dec_state_bytes / (dec_ms.mean() * 1e-3) / 1e9, 1),
            "all_GBps": round(dec_bytes / (dec_ms.mean() * 1e-3) / 1e9, 1),
            "frac_of_hbm_roof": round(dec_bytes / (dec_ms.mean() * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "us_per_step": round(dec_ms.mean() * 1e3, 2), "median_us_per_step": round(float(np.median(dec_ms)) * 1e3, 2),
            "steps_per_launch_set": steps,
        },
        "kernels": roofs,
        "dominant_kernel_by_step_time": dominant,
        "next": nxt,
    }
    checks = {"prefill_64k": pf_check, "decode": dec_check}
    del ws
    torch.cuda.empty_cache()
    if not args.no_next:
        # the other forward workloads, one after another, after the 64K workspace is released
        rec["other_workloads"], other_checks = measure_workloads(binding, configs, inputs, stream,
                                                                 dev, np, torch,
                                                                 args.cpu_1m_tokens)
        checks.update(other_checks)

    # practical HBM ceiling for context: a plain device-to-device copy
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    cev[0].record(stream)
    for i in range(5):
        dst.copy_(src)
        cev[i + 1].record(stream)
    torch.cuda.synchronize()
    copy_ms = np.mean([cev[i].elapsed_time(cev[i + 1]) for i in range(5)])
    rec["hbm_copy_reference"] = {"bytes": 2 * src.numel() * 4, "ms": round(copy_ms, 4),
                                 "GBps": round(2 * src.numel() * 4 / (copy_ms * 1e-3) / 1e9, 1)}
    del src, dst

    if not args.no_cpu_baseline:
        per, parity = cpu_leg(configs, inputs, dev, torch, np, checks, args.cpu_1m_tokens,
                              rec.get("other_workloads"), value, rec["decode"]["us_per_step"])
        top = dict(per[0])
        top["per_config"] = per
        rec["cpu_baseline"] = top
        rec["parity"] = parity
    print(json.dumps(rec), flush=True)


def measure_next(binding, inputs, ins, ws, o, ST, d, B, T, H, dk, dv, stream, dev, np, torch,
                 reps=5, every=512, draft=4, accept=2, spans=4):
    """The options built on the path, timed after the steps with HIP events:
    the prefill with bf16 output, the prefill with a state snapshot every
    `every` tokens (prefix reuse), speculative verify of `draft` tokens +
    commit of `accept` of them for the decode batch against the decode steps
    they replace (and that commit fused with the next round's verify), and
    the prefill computed span by span through the
    context-split entry points (one GPU)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    snaps = torch.empty((B, T // every, H, dk, dv), dtype=torch.float32, device=dev)

    def timed(fn, inner=1):
        # `inner` calls back to back per event pair: for kernels of a few
        # hundred microseconds the host's time in the binding would otherwise
        # fall between the start event and the launch
        ts = []
        for r in range(reps + 1):
            a, b = ev(), ev()
            a.record(stream)
            for _ in range(inner):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            if r:
                ts.append(a.elapsed_time(b) / inner)
        return float(np.mean(ts))

    snap_ms = timed(lambda: binding.kda_chunk_fwd_ex(
        ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"], ins["S0"], snapshot_every=every,
        snapshots=snaps, o=o, S_T=ST, workspace=ws))
    plain_ms = timed(lambda: binding.kda_chunk_fwd(ins["q"], ins["k"], ins["v"], ins["g"],
                                                   ins["beta"], ins["S0"], o=o, S_T=ST, workspace=ws))
    del snaps
    o16 = torch.empty(o.shape, dtype=torch.bfloat16, device=dev)
    bf16_ms = timed(lambda: binding.kda_chunk_fwd(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"],
                                                  ins["S0"], o=o16, S_T=ST, workspace=ws))
    del o16
    # the state transition of the whole sequence (dk columns, no v, no outputs)
    trans_ms = timed(lambda: binding.kda_chunk_transition(ws, B, T, H, dk, dv, torch.bfloat16))
    ctx = measure_context_split(binding, ins, B, T, H, dk, dv, spans, stream, dev, np, torch)
    N, Hd, dkd, dvd = d["S"].shape
    sp = inputs.make_forward(N, draft, Hd, dkd, dvd, "bf16", s0="zero", seed=4321, device=dev)
    Sck = d["S"].clone()
    o_sp = torch.empty((N, draft, Hd, dvd), dtype=torch.float32, device=dev)
    acc = torch.full((N,), accept, dtype=torch.int32, device=dev)
    Sw = d["S"].clone()
    ver_ms = timed(lambda: binding.kda_spec_verify(sp["q"], sp["k"], sp["v"], sp["g"], sp["beta"],
                                                   Sck, o=o_sp), inner=8)
    # each commit advances Sw by `accept` tokens: repeated commits are the same work
    com_ms = timed(lambda: binding.kda_spec_commit(sp["k"], sp["v"], sp["g"], sp["beta"], Sw, acc),
                   inner=8)
    # the next round's drafts after this one: its commit and their verify in
    # one call (each call replays the same accepted prefix onto Sf)
    sp2 = inputs.make_forward(N, draft, Hd, dkd, dvd, "bf16", s0="zero", seed=4322, device=dev)
    Sf = d["S"].clone()
    fused_ms = timed(lambda: binding.kda_spec_commit_verify(
        sp["k"], sp["v"], sp["g"], sp["beta"], acc, sp2["q"], sp2["k"], sp2["v"], sp2["g"],
        sp2["beta"], Sf, o=o_sp), inner=8)
    del sp2, Sf
    o1 = torch.empty((N, Hd, dvd), dtype=torch.float32, device=dev)
    t0 = {n: sp[n][:, 0].contiguous() for n in ("q", "k", "v", "g", "beta")}
    dec_ms = timed(lambda: binding.kda_decode_step(t0["q"], t0["k"], t0["v"], t0["g"], t0["beta"], Sw,
                                                   o=o1), inner=8)
    state = N * Hd * dkd * dvd * 4
    tok_in = N * Hd * (3 * dkd + dvd + 1) * 2           # q, k, g, v, beta per draft token
    ver_bytes = state + draft * (tok_in + N * Hd * dvd * 4)
    com_bytes = 2 * state + draft * (tok_in - N * Hd * dkd * 2)
    del sp, Sck, Sw, o_sp
    return {
        "bf16_output": {"prefill_ms": round(bf16_ms, 4), "plain_prefill_ms": round(plain_ms, 4),
                        "tokens_per_s": round(B * T / (bf16_ms * 1e-3), 1)},
        "snapshots": {"every_tokens": every, "count": T // every,
                      "bytes": B * (T // every) * H * dk * dv * 4,
                      "prefill_ms": round(snap_ms, 4), "plain_prefill_ms": round(plain_ms, 4),
                      "overhead_frac": round(snap_ms / plain_ms - 1.0, 4)},
        "transition": {"what": "kda_chunk_transition, F only, over the prepared 64K-token workload",
                       "ms": round(trans_ms, 4)},
        "context_split": ctx,
        "spec": {"requests": N, "heads": Hd, "draft_tokens": draft, "accepted": accept,
                 "verify_us": round(ver_ms * 1e3, 2),
                 "verify_GBps": round(ver_bytes / (ver_ms * 1e-3) / 1e9, 1),
                 "commit_us": round(com_ms * 1e3, 2),
                 "commit_GBps": round(com_bytes / (com_ms * 1e-3) / 1e9, 1),
                 "commit_then_verify_next_fused_us": round(fused_ms * 1e3, 2),
                 "fused_GBps": round((com_bytes + ver_bytes - state) / (fused_ms * 1e-3) / 1e9, 1),
                 "fused_vs_separate": round(fused_ms / (ver_ms + com_ms), 4),
                 "decode_step_us": round(dec_ms * 1e3, 2),
                 "verify_plus_commit_vs_decode_steps": round((ver_ms + com_ms) / (draft * dec_ms), 4)},
    }


def measure_context_split(binding, ins, B, T, H, dk, dv, spans, stream, dev, np, torch, reps=3):
    """The 64K prefill cut into `spans` equal spans and computed span by span
    on this GPU through the context-split entry points: per span kda_chunk_prep
    and kda_chunk_transition (F and E; the last span needs neither), one
    kda_state_affine_scan, then kda_chunk_state_pass per span from its entering
    state. Phase times are HIP-event measured; the result is checked against
    the plain forward."""
    L = T // spans
    xs = [{n: ins[n][:, r * L:(r + 1) * L].contiguous() for n in ("q", "k", "v", "g", "beta")}
          for r in range(spans)]
    wss = [torch.empty(binding.kda_chunk_fwd_workspace_size(B, L, H, dk, dv, 1), dtype=torch.uint8,
                       device=dev) for _ in range(spans)]
    Fs = torch.empty((spans - 1, B * H, dk, dk), dtype=torch.float32, device=dev)
    Es = torch.empty((spans - 1, B * H, dk, dv), dtype=torch.float32, device=dev)
    Sin = torch.empty((spans, B * H, dk, dv), dtype=torch.float32, device=dev)
    os_ = [torch.empty((B, L, H, dv), dtype=torch.float32, device=dev) for _ in range(spans)]
    ST = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    S0 = torch.zeros((B * H, dk, dv), dtype=torch.float32, device=dev)
    times = []
    for r in range(reps + 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        e[0].record(stream)
        for x, w in zip(xs, wss):
            binding.kda_chunk_prep(x["q"], x["k"], x["g"], x["beta"], dv, workspace=w)
        e[1].record(stream)
        for j in range(spans - 1):
            binding.kda_chunk_transition(wss[j], B, L, H, dk, dv, torch.bfloat16, v=xs[j]["v"],
                                         F=Fs[j].view(B, H, dk, dk), E=Es[j].view(B, H, dk, dv))
        e[2].record(stream)
        binding.kda_state_affine_scan(Fs, Es, S0, S=Sin)
        e[3].record(stream)
        for j in range(spans):
            binding.kda_chunk_state_pass(xs[j]["v"], wss[j], dk, Sin[j].view(B, H, dk, dv), o=os_[j],
                                         S_T=ST if j == spans - 1 else None,
                                         want_state=j == spans - 1)
        e[4].record(stream)
        torch.cuda.synchronize()
        if r:
            times.append([e[i].elapsed_time(e[i + 1]) for i in range(4)])
    t = np.mean(times, axis=0)
    o_ref, S_ref = binding.kda_chunk_fwd(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"],
                                         ins["S0"])
    o = torch.cat(os_, 1)
    torch.cuda.synchronize()
    rms = float(o_ref.double().pow(2).mean().sqrt())
    diff = float((o - o_ref).abs().max()) / rms
    diff_s = float((ST - S_ref).abs().max()) / float(S_ref.double().pow(2).mean().sqrt())
    del xs, wss, Fs, Es, Sin, os_, o, o_ref
    return {"spans": spans, "tokens_per_span": L, "prep_ms": round(float(t[0]), 4),
            "transition_ms": round(float(t[1]), 4), "scan_ms": round(float(t[2]), 4),
            "state_pass_ms": round(float(t[3]), 4), "total_ms": round(float(t.sum()), 4),
            "o_max_abs_diff_vs_plain_forward_over_rms": diff,
            "S_T_max_abs_diff_vs_plain_forward_over_rms": diff_s}


def measure_workloads(binding, configs, inputs, stream, dev, np, torch, cpu_1m_tokens):
    """kda_chunk_fwd (prep + state pass) on the forward workloads other than
    the 64K prefill, each timed with HIP events around its two launches.
    Returns the timings and host copies of the outputs for the oracle's
    check (the 1M-token workload: o over its leading tokens)."""
    out, checks = [], {}
    for key, w in (("fwd_small", configs.SMALL_FWD), ("fwd_mid", configs.MID_FWD),
                   ("prefill_1m", configs.PREFILL_1M)):
        log("workload %s" % w.name)
        ins = inputs.make_workload(w, device=dev)
        code = 0 if w.in_dtype == "f32" else 1
        ws = torch.empty(binding.kda_chunk_fwd_workspace_size(w.B, w.T, w.H, w.dk, w.dv, code),
                         dtype=torch.uint8, device=dev)
        o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device=dev)
        ST = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
        reps = 3 if w.T > 65536 else 10
        prep, pas = [], []
        for r in range(reps + 2):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            binding.kda_chunk_prep(ins["q"], ins["k"], ins["g"], ins["beta"], w.dv, workspace=ws)
            e[1].record(stream)
            binding.kda_chunk_state_pass(ins["v"], ws, w.dk, ins["S0"], o=o, S_T=ST)
            e[2].record(stream)
            torch.cuda.synchronize()
            if r >= 2:  # two warm-up runs
                prep.append(e[0].elapsed_time(e[1]))
                pas.append(e[1].elapsed_time(e[2]))
        ms = float(np.mean(np.add(prep, pas)))
        th = w.B * w.T * w.H
        es = 4 if code == 0 else 2
        flops, _ = prefill_units(w.dk, w.dv, es)
        nbytes = th * (es * (3 * w.dk + w.dv + 1) + 4 * w.dv) + w.B * w.H * w.dk * w.dv * 4 * \
            (2 if ins["S0"] is not None else 1)
        gbps = nbytes / (ms * 1e-3) / 1e9
        tflops = th * flops / (ms * 1e-3) / 1e12
        # matrix-core peak of the path's own operand type: fp32 products for
        # fp32 inputs, fp16/bf16 products for bf16 inputs
        peak = FP32_MFMA_PEAK_TFLOPS if code == 0 else BF16_MFMA_PEAK_TFLOPS
        out.append({"workload": w.name, "in_dtype": w.in_dtype, "B": w.B, "T": w.T, "H": w.H,
                    "dk": w.dk, "dv": w.dv, "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
                    "ms": round(ms, 4), "prep_ms": round(float(np.mean(prep)), 4),
                    "state_pass_ms": round(float(np.mean(pas)), 4), "timed_runs": reps,
                    "algorithmic_GBps": round(gbps, 1), "frac_of_hbm_roof": round(gbps / HBM_PEAK_GBPS, 4),
                    "algorithmic_TFLOPs": round(tflops, 3),
                    "frac_of_matrix_peak": round(tflops / peak, 5), "matrix_peak_TFLOPs": peak})
        if w.T > 65536:
            checks[key] = (o[:, :cpu_1m_tokens].cpu(), None)
        else:
            checks[key] = (o.cpu(), ST.cpu())
        del ins, ws, o, ST
        torch.cuda.empty_cache()
    return out, checks


def cpu_leg(configs, inputs, dev, torch, np, checks, cpu_1m_tokens, other, gpu_value,
            dec_us):
    """The fp64 C oracle (test infrastructure) beside every workload, timed on
    this host's cores with the same seeded inputs; its outputs check the GPU
    outputs kept from the runs above. Returns (per-config baselines, parity)."""
    from oracle import c_oracle

    to = inputs.to_oracle
    threads = c_oracle.default_threads()
    per, parity = [], {}
    gpu_rates = {w["workload"]: w["tokens_per_s"] for w in (other or [])}

    def err(x, ref):
        x = np.asarray(x, np.float64)
        rms = float(np.sqrt(np.mean(ref ** 2)))
        return float(np.abs(x - ref).max() / rms) if rms > 0 else float(np.abs(x - ref).max())

    def forward_case(key, w, ntok, sample):
        ins = inputs.make_workload(w, device=dev)
        host = {n: to(ins[n][:, :ntok].contiguous()) for n in ("q", "k", "v", "g", "beta")}
        S0 = None if ins["S0"] is None else ins["S0"].cpu().numpy()
        del ins
        torch.cuda.empty_cache()
        log("oracle: %s, %d tokens x %d heads x %d, %d threads" % (w.name, ntok, w.H, w.B, threads))
        t0 = time.perf_counter()
        o_ref, S_ref = c_oracle.fwd(host["q"], host["k"], host["v"], host["g"], host["beta"], S0,
                                    nthreads=threads)
        wall = time.perf_counter() - t0
        # per-core rate: one (b, h) on one thread, over at most 8192 tokens
        n1 = min(ntok, 8192)
        one = {n: np.ascontiguousarray(x[:1, :n1, :1]) for n, x in host.items()}
        t0 = time.perf_counter()
        c_oracle.fwd(one["q"], one["k"], one["v"], one["g"], one["beta"],
                     None if S0 is None else S0[:1, :1], nthreads=1)
        wall1 = time.perf_counter() - t0
        o_gpu, S_gpu = checks.get(key, (None, None))
        if o_gpu is not None:
            p = {"err_o_max_over_rms": err(o_gpu[:, :ntok].numpy(), o_ref), "tokens": ntok,
                 "tolerance": 1e-4 if w.in_dtype == "f32" else 2e-2}
            if S_gpu is not None and ntok == w.T:
                p["err_S_T_max_over_rms"] = err(S_gpu.numpy(), S_ref)
            parity[w.name] = p
        rate = w.B * ntok / wall
        gpu = gpu_value if key == "prefill_64k" else gpu_rates.get(w.name)
        return {"workload": w.name, "value": round(rate, 1), "unit": "tokens/s", "cores": threads,
                "kind": "oracle", "wall_s": round(wall, 3), "sample": sample,
                "gpu_tokens_per_s": gpu,
                "one_core": {"token_heads_per_s": round(n1 / wall1, 1), "wall_s": round(wall1, 3),
                             "sample": "%d tokens of one (b, h), one thread" % n1}}

    pf = configs.PREFILL_64K
    per.append(forward_case("prefill_64k", pf, pf.T, "fp64 C oracle, all %d tokens of all %d heads "
                            "of %s (o and S_T compared element-wise)" % (pf.T, pf.H, pf.name)))
    if other is not None:
        for key, w in (("fwd_small", configs.SMALL_FWD), ("fwd_mid", configs.MID_FWD)):
            per.append(forward_case(key, w, w.T, "fp64 C oracle, the whole workload %s" % w.name))
        w = configs.PREFILL_1M
        n = min(cpu_1m_tokens, w.T)
        per.append(forward_case("prefill_1m", w, n, "fp64 C oracle, the first %d of %d tokens of all "
                                "%d heads of %s (o compared on those tokens)" % (n, w.T, w.H, w.name)))
    # decode: 64 single-token steps over all (request, head) units
    dc = configs.DECODE
    d = inputs.make_workload(dc, device=dev)
    host = {n: to(d[n]) for n in ("q", "k", "v", "g", "beta")}
    S = d["S"].cpu().numpy().astype(np.float64)
    del d
    torch.cuda.empty_cache()
    log("oracle: %s, %d threads" % (dc.name, threads))
    t0 = time.perf_counter()
    outs = []
    for s in range(dc.T):
        o_s, S = c_oracle.fwd(host["q"][s][:, None], host["k"][s][:, None], host["v"][s][:, None],
                              host["g"][s][:, None], host["beta"][s][:, None], S, nthreads=threads)
        outs.append(o_s[:, 0])
    wall = time.perf_counter() - t0
    o_gpu, S_gpu = checks["decode"]
    parity[dc.name] = {"err_o_max_over_rms": err(o_gpu.numpy(), np.stack(outs)),
                       "err_S_max_over_rms": err(S_gpu.numpy(), S), "steps": dc.T, "tolerance": 1e-4}
    units = dc.B * dc.H
    t0 = time.perf_counter()
    S1 = np.zeros((1, dc.H, dc.dk, dc.dv))
    for s in range(dc.T):
        _, S1 = c_oracle.fwd(host["q"][s][:1, None], host["k"][s][:1, None], host["v"][s][:1, None],
                             host["g"][s][:1, None], host["beta"][s][:1, None], S1, nthreads=1)
    wall1 = time.perf_counter() - t0
    per.append({"workload": dc.name, "value": round(units * dc.T / wall, 1),
                "unit": "request-head steps/s", "cores": threads, "kind": "oracle",
                "wall_s": round(wall, 3),
                "sample": "fp64 C oracle, all %d steps of all %d requests x %d heads (o of every step "
                          "and the final states compared element-wise)" % (dc.T, dc.B, dc.H),
                "gpu_request_head_steps_per_s": round(units / (dec_us * 1e-6), 1),
                "one_core": {"request_head_steps_per_s": round(dc.H * dc.T / wall1, 1),
                             "wall_s": round(wall1, 3),
                             "sample": "%d steps of one request (%d heads), one thread" % (dc.T, dc.H)}})
    return per, parity


if __name__ == "__main__":
    main()
