"""Benchmark of the block-draft readout hot path on one MI355X.

One step = one block-step over one batch: dflash_fuse_fc (S1) ->
dspark_lm_head + dspark_markov_argmax (S2 + S3; dspark_draft_block is exactly
these two calls) -> spec_verify_greedy (S4).  Inputs cycle through a pool of
pre-generated seeded steps that are resident in HBM before timing starts.

Prints ONE JSON line: block-steps/s over K back-to-back steps (the headline),
per-step medians and 10th/90th percentiles with the pool rotating, with the
MALL flushed before each step and with one step repeated (warm), the roofline
of the dominant kernel (the LM-head GEMM, timed with HIP events on its launch
stream), each stage's time, algorithmic bytes, GB/s and fraction of the HBM
peak, and the CPU oracle timed on a bounded sample of the same workload (plus
one-thread figures of two small workloads).
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


GEMM_SOURCES = ("gemm.hip", "gemm_kernels.h", "gemm_ns.h", "gemm_ns_bf16.hip",
                "gemm_ns_packed.hip", "gemm_ns_pair_a.hip", "gemm_ns_pair_b.hip",
                "gemm_ns_pair_packed.hip", "pack.hip", "bdr_device.h", "gemm_plan.h")
GEMM_FP8_SOURCES = ("gemm_fp8.hip", "gemm_ns.h", "gemm_ns_fp8.hip", "gemm_ns_fp8_reg.hip",
                    "gemm_kernels.h", "bdr_device.h", "gemm_plan.h")


def kernel_source_hash(sources=GEMM_SOURCES) -> str:
    """Hash of the code (comments and whitespace removed) of the sources that
    define the LM-head GEMM kernels."""
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "block_draft_readout_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, weights: str = "native", kernel: str = "lm_head_gemm"):
    """HBM bytes per launch of the dominant kernel (the LM head, or the fc and
    the LM head in one launch: kernel="fc_lm_head_gemm") from the committed
    rocprofv3 counter summary of that weight format (native, packed, fp8), or
    None when the summary is missing or the kernel has changed since."""
    fp8 = weights == "fp8"
    name = (f"{kernel}_{weights}_{workload}_pmc.md" if weights != "native"
            else f"{kernel}_{workload}_pmc.md")
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    want = kernel_source_hash(GEMM_FP8_SOURCES if fp8 else GEMM_SOURCES)
    if not m_hash or not m_bytes or m_hash.group(1) != want:
        return None
    return float(m_bytes.group(1))


class Step:
    """Pre-bound C-ABI calls of one pool slot (pointers resolved once)."""

    def __init__(self, L, w, dt, g, slot, bufs, stream, sample=None, fp8=False, wdt=None):
        self.L, self.w, self.dt, self.g, self.s, self.b = L, w, dt, g, slot, bufs
        self.sample = sample      # None: greedy; else (temperature, seed)
        self.fp8 = fp8            # fc and LM head weights as E4M3 codes + row scales
        self.wdt = dt if wdt is None else wdt   # dtype of the calls with fc / LM-head weights
        self.stream = stream
        self.fc_stream = stream   # the fc may run on a second stream (see --overlap)
        self.taps = (C.c_void_p * w.n_taps)(*[t.data_ptr() for t in slot["taps"]])
        self.prev = slot["prev0"].data_ptr()   # Markov context of position 0 (see --closed-loop)
        # each slot may hold its own copy of the Markov weights (same values), so
        # that consecutive steps find none of their inputs in the MALL
        self.w1 = slot.get("w1", g["w1"]).data_ptr()
        self.w2 = slot.get("w2", g["w2"]).data_ptr()
        self.status = None        # device int32 for the Markov calls' status word

    def fc(self):
        w, b = self.w, self.b
        if self.fp8:
            return self.L.dflash_fuse_fc_fp8(self.taps, w.n_taps, w.rows, w.hidden,
                                             self.g["fc_q"].data_ptr(), self.g["fc_scale"].data_ptr(),
                                             b["F"].data_ptr(), b["ws_fc"], b["ws_fc_n"],
                                             self.fc_stream)
        return self.L.dflash_fuse_fc(self.taps, w.n_taps, w.rows, w.hidden, self.wdt,
                                     self.g["fc_w"].data_ptr(), b["F"].data_ptr(),
                                     b["ws_fc"], b["ws_fc_n"], self.fc_stream)

    def fc_lm(self):
        """S1 and S2 in one call (one launch on the batched workloads)."""
        w, b = self.w, self.b
        return self.L.dflash_fuse_fc_lm_head(self.taps, w.n_taps, w.rows, w.hidden, self.wdt,
                                             self.g["fc_w"].data_ptr(), b["F"].data_ptr(),
                                             self.s["draft_hidden"].data_ptr(), w.batch * w.k,
                                             w.vocab, self.g["lm_w"].data_ptr(),
                                             b["logits"].data_ptr(), b["ws_fcl"], b["ws_fcl_n"],
                                             self.stream)

    def lm_head(self):
        w = self.w
        if self.fp8:
            return self.L.dspark_lm_head_fp8(self.s["draft_hidden"].data_ptr(), w.batch * w.k,
                                             w.hidden, w.vocab, self.g["lm_q"].data_ptr(),
                                             self.g["lm_scale"].data_ptr(),
                                             self.b["logits"].data_ptr(), self.stream)
        return self.L.dspark_lm_head(self.s["draft_hidden"].data_ptr(), w.batch * w.k, w.hidden,
                                     w.vocab, self.wdt, self.g["lm_w"].data_ptr(),
                                     self.b["logits"].data_ptr(), self.stream)

    def markov(self):
        w, b = self.w, self.b
        if self.sample is not None:
            T, seed = self.sample
            conf = self.s.get("conf")
            th = float("nan") if w.threshold is None else w.threshold
            return self.L.dspark_markov_sample(
                b["logits"].data_ptr(), w.batch, w.k, w.vocab, self.dt, self.w1, self.w2,
                w.rank, self.prev, T, seed, b["d"].data_ptr(), b["x"].data_ptr(),
                None if conf is None else conf.data_ptr(), th, self.status,
                b["ws_ms"], b["ws_ms_n"], self.stream)
        return self.L.dspark_markov_argmax(b["logits"].data_ptr(), w.batch, w.k, w.vocab, self.dt,
                                           self.w1, self.w2, w.rank, self.prev, b["d"].data_ptr(),
                                           self.status, b["ws_m"], b["ws_m_n"], self.stream)

    def draft_block(self):
        w, b = self.w, self.b
        if self.fp8:     # the same two calls with the fp8 LM head
            rc = self.lm_head()
            return rc if rc != 0 else self.markov()
        return self.L.dspark_draft_block(self.s["draft_hidden"].data_ptr(), w.batch, w.k,
                                         w.hidden, w.vocab, self.wdt, self.g["lm_w"].data_ptr(),
                                         self.w1, self.w2, w.rank,
                                         self.s["prev0"].data_ptr(), b["d"].data_ptr(),
                                         b["logits"].data_ptr(), self.status, b["ws_m"],
                                         b["ws_m_n"], self.stream)

    def verify(self):
        w, b = self.w, self.b
        conf = self.s.get("conf")
        th = float("nan") if w.threshold is None else w.threshold
        if self.sample is not None:
            T, seed = self.sample
            return self.L.spec_verify_sample(
                self.s["Y"].data_ptr(), self.dt, w.batch, w.k, w.vocab, b["d"].data_ptr(),
                b["x"].data_ptr(), None if conf is None else conf.data_ptr(), th, T, seed,
                b["bl"].data_ptr(), b["acc_len"].data_ptr(), b["bonus"].data_ptr(),
                b["acc"].data_ptr(), b["prop"].data_ptr(), b["ws_vs"], b["ws_vs_n"], self.stream)
        return self.L.spec_verify_greedy(
            self.s["Y"].data_ptr(), self.dt, w.batch, w.k, w.vocab, b["d"].data_ptr(),
            None if conf is None else conf.data_ptr(), th, b["bl"].data_ptr(),
            b["acc_len"].data_ptr(), b["bonus"].data_ptr(), b["targ"].data_ptr(),
            b["acc"].data_ptr(), b["prop"].data_ptr(), b["ws_v"], b["ws_v_n"], self.stream)


    def commit(self, next_prev):
        w, b = self.w, self.b
        return self.L.spec_commit(b["d"].data_ptr(), b["acc_len"].data_ptr(), b["bonus"].data_ptr(),
                                  b["bl"].data_ptr(), w.batch, w.k, next_prev,
                                  b["emitted"].data_ptr(), b["draft_list"].data_ptr(),
                                  b["row_index"].data_ptr(), b["row_count"].data_ptr(),
                                  b["row_offsets"].data_ptr(), self.stream)

    def fc_rows(self):
        w, b = self.w, self.b
        if self.fp8:
            return self.L.dflash_fuse_fc_rows_fp8(
                self.taps, w.n_taps, w.rows, w.hidden, b["row_index"].data_ptr(),
                b["row_count"].data_ptr(), w.rows, self.g["fc_q"].data_ptr(),
                self.g["fc_scale"].data_ptr(), b["F"].data_ptr(), b["ws_fcr"], b["ws_fcr_n"],
                self.stream)
        return self.L.dflash_fuse_fc_rows(self.taps, w.n_taps, w.rows, w.hidden, self.wdt,
                                          b["row_index"].data_ptr(), b["row_count"].data_ptr(),
                                          w.rows, self.g["fc_w"].data_ptr(), b["F"].data_ptr(),
                                          b["ws_fcr"], b["ws_fcr_n"], self.stream)


_HIP = None


def hip_runtime():
    """The HIP runtime through ctypes (event calls torch does not expose)."""
    global _HIP
    if _HIP is None:
        h = C.CDLL("libamdhip64.so")
        h.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        h.hipStreamWaitEvent.argtypes = [C.c_void_p, C.c_void_p, C.c_uint]
        h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        _HIP = h
    return _HIP


HIP_EVENT_DISABLE_TIMING = 0x2
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def hip_event(flags):
    ev = C.c_void_p()
    rc = hip_runtime().hipEventCreateWithFlags(C.byref(ev), flags)
    if rc != 0:
        raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
    return ev


class LaunchTimer:
    """Start/stop HIP events around launches on one stream, created without the
    system-scope fence, so the stop stamp is not stretched by a flush for host
    visibility (the default event record adds ~3 us to a 227 us kernel)."""

    def __init__(self, n):
        self.ev = [(hip_event(HIP_EVENT_DISABLE_SYSTEM_FENCE), hip_event(HIP_EVENT_DISABLE_SYSTEM_FENCE))
                   for _ in range(n)]

    def start(self, i, stream_ptr):
        if hip_runtime().hipEventRecord(self.ev[i][0], stream_ptr) != 0:
            raise RuntimeError("hipEventRecord failed")

    def stop(self, i, stream_ptr):
        if hip_runtime().hipEventRecord(self.ev[i][1], stream_ptr) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, i):
        out = C.c_float()
        if hip_runtime().hipEventElapsedTime(C.byref(out), self.ev[i][0], self.ev[i][1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)


def check(rc, what):
    if rc != 0:
        import block_draft_readout_amd as bdr
        raise RuntimeError(f"{what} failed ({rc}): {bdr.lib().bdr_last_error().decode()}")


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(w, W, slot_host, budget_s=10.0, max_steps=30, sample=None, fp8=False):
    """The oracle, as it stands, on whole block-steps of the workload: repeats
    the step of pool slot 0 until about ``budget_s`` seconds of CPU work.
    ``sample`` = (temperature, seed) times the probabilistic path instead;
    ``fp8`` times the fp8-weight fc and LM head.  ``cores`` is the number of
    threads the oracle's BLAS calls use (its Python loops run on one)."""
    import oracle
    from oracle import fp8 as ofp8
    from oracle import sampling
    blas = _blas_threads()
    n = 0
    t0 = time.perf_counter()
    while True:
        if fp8:
            ofp8.fuse_fc_fp8(slot_host["taps"], W["fc_q"], W["fc_scale"], w.dtype)
            Z = ofp8.lm_head_fp8(slot_host["draft_hidden"], W["lm_q"], W["lm_scale"], w.dtype)
            if sample is None:
                d, _ = oracle.semi_ar_argmax(Z, W["w1"], W["w2"], slot_host["prev0"], w.dtype)
                Lb = oracle.truncate_by_confidence(slot_host["conf"], w.threshold, w.batch, w.k)
                oracle.verify_greedy(d, oracle.target_argmax(slot_host["Y"], w.dtype, Lb), Lb)
            else:
                sampling.block_step_sample(w.dtype, Z, W["w1"], W["w2"], slot_host["prev0"],
                                           slot_host["Y"], sample[0], sample[1],
                                           confidence=slot_host["conf"], threshold=w.threshold)
        elif sample is None:
            oracle.block_step(w.dtype, slot_host["taps"], W["fc_w"], slot_host["draft_hidden"],
                              W["lm_w"], W["w1"], W["w2"], slot_host["prev0"],
                              target_logits=slot_host["Y"], confidence=slot_host["conf"],
                              threshold=w.threshold)
        else:
            oracle.fuse_fc(slot_host["taps"], W["fc_w"], w.dtype)
            Z = oracle.lm_head(slot_host["draft_hidden"], W["lm_w"], w.dtype)
            sampling.block_step_sample(w.dtype, Z, W["w1"], W["w2"], slot_host["prev0"],
                                       slot_host["Y"], sample[0], sample[1],
                                       confidence=slot_host["conf"], threshold=w.threshold)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or n >= max_steps:
            break
    return {"value": n / dt, "unit": "block-steps/s", "cores": int(blas), "kind": "oracle",
            "sample": f"{n} full {'probabilistic' if sample else 'greedy'} block-steps of "
                      f"{'(fp8 weights) ' if fp8 else ''}"
                      f"{w.name} (S1-S4, all {w.batch} rows) in "
                      f"{dt:.1f} s on the host; numpy float64 BLAS on {blas} threads "
                      f"(host affinity {len(os.sched_getaffinity(0))} cores)"}


def cpu_one_thread(names=("tiny", "qwen27b_b1"), budget_s=4.0):
    """The oracle on one thread (BLAS limited to 1) for small workloads: greedy
    block-steps/s on a bounded sample of each (targets planted on the oracle's
    own draft)."""
    import oracle
    import workloads
    from workloads import synth
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        return None
    out = {}
    with threadpool_limits(limits=1):
        for name in names:
            w = workloads.get(name)
            W = synth.make_weights(w)
            s = synth.make_step(w, 0)
            ref = oracle.block_step(w.dtype, s["taps"], W["fc_w"], s["draft_hidden"], W["lm_w"],
                                    W["w1"], W["w2"], s["prev0"])
            Y = synth.plant_targets(w, 0, s["noise"], ref["draft_tokens"])["target_logits"]
            conf = synth.make_confidence(w, 0)
            n, t0 = 0, time.perf_counter()
            while True:
                oracle.block_step(w.dtype, s["taps"], W["fc_w"], s["draft_hidden"], W["lm_w"],
                                  W["w1"], W["w2"], s["prev0"], target_logits=Y, confidence=conf,
                                  threshold=w.threshold)
                n += 1
                dt = time.perf_counter() - t0
                if dt >= budget_s or n >= 200:
                    break
            out[name] = {"value": n / dt, "unit": "block-steps/s", "cores": 1,
                         "sample": f"{n} greedy block-steps in {dt:.1f} s"}
            del W
    return out


def fc_only(args, w, L, bdr, synth, torch, dev):
    """Times dflash_fuse_fc alone on args.fc_rows rows (taps and fc_w of the
    workload's shape, synthetic N(0, 1) / N(0, 1/fan_in)); one JSON line."""
    rows, H, T = args.fc_rows, w.hidden, w.n_taps
    dt = bdr.BDR_BF16 if w.dtype == "bf16" else bdr.BDR_F32

    def up(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    hc = args.hc
    if hc > 1:
        # captured layer outputs with hc streams, memory [rows, hc, H]; the taps
        # are their averages (dflash_hc_average), then the fc runs on them
        cap = [up(synth.store(synth.normal_f32((rows, hc, H), (w.cid, 6, 0, t)), w.dtype))
               for t in range(T)]
        taps = [torch.empty((rows, H), dtype=cap[0].dtype, device=dev) for _ in range(T)]
        cap_arr = (C.c_void_p * T)(*[c.data_ptr() for c in cap])
        tap_arr = (C.c_void_p * T)(*[t.data_ptr() for t in taps])
    else:
        taps = [up(synth.store(synth.normal_f32((rows, H), (w.cid, 5, 0, t)), w.dtype))
                for t in range(T)]
    fc_w = up(synth.store(synth.normal_f32((H, T * H), (w.cid, 0, 0, 0), math.sqrt(1.0 / (T * H))),
                          w.dtype))
    out = torch.empty((rows, H), dtype=fc_w.dtype, device=dev)
    nws = L.dflash_fuse_fc_workspace_bytes(rows, H, T, dt)
    wst = torch.zeros(nws + 256, dtype=torch.uint8, device=dev)
    wsp = C.c_void_p((wst.data_ptr() + 255) & ~255)
    arr = (C.c_void_p * T)(*[t.data_ptr() for t in taps])
    stream = torch.cuda.current_stream(dev)
    sp = C.c_void_p(stream.cuda_stream)

    def average():
        check(L.dflash_hc_average(cap_arr, T, hc, rows, H, H, hc * H, dt, tap_arr, sp),
              "dflash_hc_average")

    def run():
        check(L.dflash_fuse_fc(arr, T, rows, H, dt, fc_w.data_ptr(), out.data_ptr(), wsp, nws, sp),
              "dflash_fuse_fc")

    for _ in range(args.warmup):
        if hc > 1:
            average()
        run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    hevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for (a, b), (ha, hb) in zip(evs, hevs):
        if hc > 1:
            ha.record(stream)
            average()
            hb.record(stream)
        a.record(stream)
        run()
        b.record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    per = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    hc_info = None
    if hc > 1:
        hper = float(np.mean([a.elapsed_time(b) for a, b in hevs]))
        hbytes = T * rows * H * (hc + 1) * (2 if w.dtype == "bf16" else 4)
        hgbs = hbytes / (hper * 1e-3) / 1e9
        log(f"hc average ({hc} streams, {T} taps): {hper * 1e3:.1f} us = {hgbs:.0f} GB/s")
        hc_info = {"streams": hc, "layout": "[rows, hc, H]", "avg_launch_us": hper * 1e3,
                   "algorithmic_bytes_per_launch": hbytes, "achieved_GBs": hgbs,
                   "frac_of_hbm_peak": hgbs / HBM_PEAK_GBS}
    flops = 2.0 * rows * H * T * H
    tflops = flops / (per * 1e-3) / 1e12
    esz = 2 if w.dtype == "bf16" else 4
    nbytes = (rows * T * H + H * T * H + rows * H) * esz
    log(f"fc rows={rows} H={H} T={T}: {per * 1e3:.1f} us per launch, {tflops:.0f} TFLOP/s")
    print(json.dumps({
        "metric": "drafter fc TFLOP/s (prefill-shaped rows)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"fc {rows} x {T}x{H} -> {H} ({w.name} shape)"
                               + (f", taps averaged over {hc} hc streams" if hc > 1 else ""),
                   "rows": rows, "hidden": H, "n_taps": T, "hc_streams": hc},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "tiled GEMM (dflash_fuse_fc)", "avg_launch_us": per * 1e3,
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": nbytes},
        "hc_average": hc_info,
        "cpu_baseline": None}), flush=True)


def _pct(xs):
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="adaptive_b16")
    ap.add_argument("--pool", type=int, default=8)
    ap.add_argument("--graph", action="store_true", help="replay HIP graphs of whole steps")
    ap.add_argument("--overlap", choices=("auto", "fused", "none", "lm", "chain"), default="auto",
                    help="auto: whichever of fused and chain is faster over 20 warm steps; "
                         "fused: the fc and the LM head in one call (dflash_fuse_fc_lm_head); "
                         "otherwise the fc runs on its own: in order (none), or on a second "
                         "stream concurrently with the LM head (lm) or with the Markov chain "
                         "and verification (chain); the fc output feeds the next step's "
                         "drafter, not S2-S4 of this step")
    ap.add_argument("--draft", choices=("greedy", "sample"), default="greedy",
                    help="greedy drafting + exact-match verification, or probabilistic "
                         "drafting + rejection-sampling verification")
    ap.add_argument("--temperature", type=float, default=1.0, help="sampling temperature")
    ap.add_argument("--closed-loop", action="store_true",
                    help="chain the steps on the device: each step's Markov context is the previous "
                         "step's bonus token, and the fc runs after verification on the accepted "
                         "rows only (LM head, draft, verify, commit, fc in order)")
    ap.add_argument("--fc-rows", type=int, default=0,
                    help="time the drafter fc alone on this many rows (the prefill-shaped, "
                         "MFMA-bound fc) with the workload's H and taps, instead of block-steps")
    ap.add_argument("--weights", choices=("auto", "native", "packed", "fp8"), default="auto",
                    help="native: fc and LM head weights in the workload's dtype, row-major; "
                         "packed: bf16 fc and LM head weights in the packed layout "
                         "(bdr_pack_weight, done once before timing); fp8: E4M3 codes with "
                         "one fp32 scale per row (bf16 workloads); auto: packed for bf16 "
                         "workloads whose LM head has more than 16 rows, else native")
    ap.add_argument("--hc", type=int, default=1,
                    help="with --fc-rows: average each tap over this many hyper-connection "
                         "streams (dflash_hc_average) before the fc; both are timed")
    ap.add_argument("--shared-markov", action="store_true",
                    help="one copy of the Markov weights for every pool slot (by default each "
                         "slot has its own copy, so consecutive steps share no input)")
    ap.add_argument("--dist-steps", type=int, default=50,
                    help="steps of each per-step timing phase (rotated, cold, warm)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, copy a 1 GiB buffer 3 times (counter calibration)")
    args = ap.parse_args()

    if args.closed_loop and args.graph:
        print(json.dumps({"error": "--closed-loop runs eagerly (no --graph)"}))
        sys.exit(2)
    fp8 = args.weights == "fp8"
    packed = args.weights == "packed"
    if (fp8 or packed) and args.fc_rows > 0:
        print(json.dumps({"error": f"--weights {args.weights} times block-steps (not --fc-rows)"}))
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import block_draft_readout_amd as bdr
    import workloads
    from workloads import synth

    w = workloads.get(args.workload)
    if args.weights == "auto":
        # the packed layout serves the batched (row-split) GEMMs; up to 16 rows the
        # row-major layout's one-sequence kernel is the faster one
        args.weights = ("packed" if w.dtype == "bf16" and w.batch * w.k > 16 and args.fc_rows == 0
                        else "native")
        packed = args.weights == "packed"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = bdr.lib()
    if args.fc_rows > 0:
        fc_only(args, w, L, bdr, synth, torch, dev)
        return
    dt = bdr.BDR_BF16 if w.dtype == "bf16" else bdr.BDR_F32
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    if (fp8 or packed) and w.dtype != "bf16":
        print(json.dumps({"error": f"--weights {args.weights} needs a bf16 workload"}))
        sys.exit(2)
    wdt = bdr.BDR_BF16_PACKED if packed else dt
    if args.overlap == "auto" and (fp8 or args.closed_loop or args.graph):
        # the fused call takes bf16 weights; a closed loop runs in order; graphs are
        # captured before any timing
        args.overlap = "chain"
    if fp8 and args.overlap == "fused":
        args.overlap = "chain"      # the fused call takes bf16 weights
    t0 = time.time()
    W = synth.make_weights_fp8(w) if fp8 else synth.make_weights(w)
    g = {k: up(v) for k, v in W.items()}
    if packed:      # the load-time copy; the row-major weights are not kept
        g["fc_w"], g["lm_w"] = bdr.pack_weight(g["fc_w"]), bdr.pack_weight(g["lm_w"])
        torch.cuda.synchronize()
    log(f"{w.describe()}: weights ready in {time.time() - t0:.1f}s")

    stream = torch.cuda.current_stream(dev)
    sptr = C.c_void_p(stream.cuda_stream)

    def ws(n):
        if n == 0:
            return None, 0, None
        t = torch.zeros(n + 256, dtype=torch.uint8, device=dev)
        p = (t.data_ptr() + 255) & ~255
        return C.c_void_p(p), n, t

    B, k, V, H = w.batch, w.k, w.vocab, w.hidden
    keep = []
    bufs = {"F": torch.empty((w.rows, H), dtype=tdt, device=dev),
            "logits": torch.empty((B, k, V), dtype=torch.float32, device=dev),
            "d": torch.empty((B, k), dtype=torch.int32, device=dev),
            "bl": torch.empty(B, dtype=torch.int32, device=dev),
            "acc_len": torch.empty(B, dtype=torch.int32, device=dev),
            "bonus": torch.empty(B, dtype=torch.int32, device=dev),
            "targ": torch.empty((B, k + 1), dtype=torch.int32, device=dev),
            "acc": torch.zeros(k, dtype=torch.int64, device=dev),
            "prop": torch.zeros(k, dtype=torch.int64, device=dev),
            "status": torch.full((1,), -1, dtype=torch.int32, device=dev)}
    sampling = args.draft == "sample"
    if sampling:
        bufs["x"] = torch.empty((B, k, V), dtype=torch.float32, device=dev)
    if args.closed_loop:
        for name, shp in (("prev_a", (B,)), ("prev_b", (B,)), ("emitted", (B, k + 1)),
                          ("draft_list", (B, k)), ("row_index", (B * (k + 1),)), ("row_count", (1,)),
                          ("row_offsets", (B + 1,))):
            bufs[name] = torch.zeros(shp, dtype=torch.int32, device=dev)
    for key, n in (("ws_fc", L.dflash_fuse_fc_fp8_workspace_bytes(w.rows, H, w.n_taps) if fp8
                     else L.dflash_fuse_fc_workspace_bytes(w.rows, H, w.n_taps, wdt)),
                   ("ws_m", L.dspark_markov_workspace_bytes(B, k)),
                   ("ws_fcl", 0 if fp8 else L.dflash_fuse_fc_lm_head_workspace_bytes(
                       w.rows, H, w.n_taps, B * k, V, wdt)),
                   ("ws_v", L.spec_verify_workspace_bytes(B, k, V)),
                   ("ws_ms", L.dspark_markov_sample_workspace_bytes(B, k, V) if sampling else 0),
                   ("ws_vs", L.spec_verify_sample_workspace_bytes(B, k, V) if sampling else 0),
                   ("ws_fcr", (L.dflash_fuse_fc_rows_fp8_workspace_bytes(w.rows, H, w.n_taps) if fp8
                               else L.dflash_fuse_fc_rows_workspace_bytes(w.rows, H, w.n_taps, wdt))
                    if args.closed_loop else 0)):
        p, n2, t = ws(n)
        bufs[key], bufs[key + "_n"] = p, n2
        keep.append(t)

    # pool of steps resident in HBM; targets planted on this path's own draft
    t0 = time.time()
    slots, host0 = [], None
    verify_bytes = []
    x_positions = []     # sampling: (row, position) pairs whose x is written (j < L_b)
    es = 2 if w.dtype == "bf16" else 4
    for p in range(args.pool):
        s = synth.make_step(w, p)
        slot = {"taps": [up(t) for t in s["taps"]], "draft_hidden": up(s["draft_hidden"]),
                "prev0": up(s["prev0"])}
        if not args.shared_markov:
            slot["w1"], slot["w2"] = g["w1"].clone(), g["w2"].clone()
        conf = synth.make_confidence(w, p)
        slot["conf"] = None if conf is None else up(conf)
        st = Step(L, w, dt, g, slot, bufs, sptr,
                  sample=(args.temperature, 0x5EED0000 + p) if sampling else None, fp8=fp8,
                  wdt=wdt)
        check(st.draft_block(), "dspark_draft_block")
        if sampling:   # plant the targets on this step's sampled draft
            check(st.markov(), "dspark_markov_sample")
        torch.cuda.synchronize()
        d_host = bufs["d"].cpu().numpy()
        Y = synth.plant_targets(w, p, s["noise"], d_host)["target_logits"]
        slot["Y"] = up(Y)
        check(st.verify(), "verification")
        torch.cuda.synchronize()
        # verification reads the rows of the (confidence-truncated) blocks only
        verify_bytes.append(int((bufs["bl"].cpu().numpy().astype(np.int64) + 1).sum()) * V * es)
        x_positions.append(int(bufs["bl"].cpu().numpy().astype(np.int64).sum()))
        slots.append(st)
        if p == 0:
            host0 = {"taps": s["taps"], "draft_hidden": s["draft_hidden"], "prev0": s["prev0"],
                     "Y": Y, "conf": conf}
    bufs["acc"].zero_()
    bufs["prop"].zero_()
    log(f"pool of {args.pool} steps ready in {time.time() - t0:.1f}s")

    stream2 = torch.cuda.Stream(dev)          # default priority
    s2ptr = C.c_void_p(stream2.cuda_stream)
    # fork / join events for the fc beside the chain: device-side ordering only
    # (nothing the host reads crosses them), so they are created without the
    # system-scope fence that a default event record carries (-4 us per step)
    hip = hip_runtime()
    ev_fork = hip_event(HIP_EVENT_DISABLE_TIMING | HIP_EVENT_DISABLE_SYSTEM_FENCE)
    ev_join = hip_event(HIP_EVENT_DISABLE_TIMING | HIP_EVENT_DISABLE_SYSTEM_FENCE)

    def record(ev, stream_ptr):
        if hip.hipEventRecord(ev, stream_ptr) != 0:
            raise RuntimeError("hipEventRecord failed")

    def wait(stream_ptr, ev):
        if hip.hipStreamWaitEvent(stream_ptr, ev, 0) != 0:
            raise RuntimeError("hipStreamWaitEvent failed")

    loop_state = {"cur": "prev_a"}
    if args.closed_loop:
        bufs["prev_a"].copy_(slots[0].s["prev0"])
        torch.cuda.synchronize()

    def run_step(st):
        if args.closed_loop:
            cur = loop_state["cur"]
            nxt = "prev_b" if cur == "prev_a" else "prev_a"
            st.prev = bufs[cur].data_ptr()
            check(st.lm_head(), "dspark_lm_head")
            check(st.markov(), "drafting")
            check(st.verify(), "verification")
            check(st.commit(bufs[nxt].data_ptr()), "spec_commit")
            check(st.fc_rows(), "dflash_fuse_fc_rows")
            st.prev = st.s["prev0"].data_ptr()
            loop_state["cur"] = nxt
            return
        if args.overlap == "fused":
            check(st.fc_lm(), "dflash_fuse_fc_lm_head")
            check(st.markov(), "drafting")
            check(st.verify(), "verification")
            return
        if args.overlap == "none":
            check(st.fc(), "dflash_fuse_fc")
            check(st.lm_head(), "dspark_lm_head")
            check(st.markov(), "drafting")
            check(st.verify(), "verification")
            return
        main = C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        fc_ptr = st.fc_stream
        st.fc_stream = s2ptr
        if args.overlap == "chain":
            check(st.lm_head(), "dspark_lm_head")
        record(ev_fork, main)
        wait(s2ptr, ev_fork)
        check(st.fc(), "dflash_fuse_fc")
        record(ev_join, s2ptr)
        if args.overlap == "lm":
            check(st.lm_head(), "dspark_lm_head")
        check(st.markov(), "drafting")
        check(st.verify(), "verification")
        wait(main, ev_join)
        st.fc_stream = fc_ptr

    graphs = None
    if args.graph:
        graphs = []
        for st in slots:  # warm once eagerly (device checks, caches), then capture
            run_step(st)
        torch.cuda.synchronize()
        for st in slots:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                cs = C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
                st.stream = st.fc_stream = cs
                run_step(st)
            st.stream = st.fc_stream = sptr
            graphs.append(gr)

    def step_i(i):
        if graphs is not None:
            graphs[i % len(graphs)].replay()
        else:
            run_step(slots[i % len(slots)])

    # the schedule of the fc: one launch with the LM head, or beside the chain on a
    # second stream -- whichever runs the whole step faster here (the two are
    # timed in turn, four rounds of 10 steps each, after 10 warm steps of each)
    overlap_choice = None
    if args.overlap == "auto":
        times = {"fused": 0.0, "chain": 0.0}
        for rnd in range(5):
            for cand in ("fused", "chain"):
                args.overlap = cand
                ea = torch.cuda.Event(enable_timing=True)
                eb = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                ea.record(stream)
                for i in range(10):
                    step_i(i)
                eb.record(stream)
                torch.cuda.synchronize()
                if rnd > 0:
                    times[cand] += ea.elapsed_time(eb) / 40 * 1e3
        args.overlap = min(times, key=times.get)
        overlap_choice = {k: round(v, 1) for k, v in times.items()}
        log(f"fc schedule: {args.overlap} (us per step over 40 warm steps: {overlap_choice})")

    for i in range(args.warmup):
        step_i(i)
    torch.cuda.synchronize()

    # phase 1 (the headline): K whole steps back to back, cycling the pool
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step_i(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # phase 2: per-step distributions (HIP events around each step on the main
    # stream; the fc joins it before the stop stamp)
    sptr_now = C.c_void_p(stream.cuda_stream)
    nd = max(1, args.dist_steps)
    flush = torch.ones(1 << 27, dtype=torch.int64, device=dev)      # 1 GiB
    dist = {}
    for mode in ("rotated", "cold", "warm"):
        tm = LaunchTimer(nd)
        torch.cuda.synchronize()
        for i in range(nd):
            if mode == "cold":        # 1 GiB read between steps: the MALL holds none of the step
                torch.amax(flush)
            tm.start(i, sptr_now)
            step_i(0 if mode == "warm" else i)
            tm.stop(i, sptr_now)
        torch.cuda.synchronize()
        dist[mode] = _pct([tm.ms(i) * 1e3 for i in range(nd)])
    del flush
    log("per-step us (median/p10/p90): " + ", ".join(
        f"{m} {d['median']:.1f}/{d['p10']:.1f}/{d['p90']:.1f}" for m, d in dist.items()))

    # phase 3: the same steps in stream order, HIP events around each launch of the
    # dominant kernel (the fc and the LM head in one launch when fused, else the LM head)
    fused = args.overlap == "fused" and not args.closed_loop
    lm_t = LaunchTimer(args.steps)
    torch.cuda.synchronize()
    for i in range(args.steps):
        st = slots[i % len(slots)]
        if fused:
            lm_t.start(i, sptr_now)
            check(st.fc_lm(), "dflash_fuse_fc_lm_head")
            lm_t.stop(i, sptr_now)
        else:
            check(st.fc(), "dflash_fuse_fc")
            lm_t.start(i, sptr_now)
            check(st.lm_head(), "dspark_lm_head")
            lm_t.stop(i, sptr_now)
        check(st.markov(), "drafting")
        check(st.verify(), "verification")
    torch.cuda.synchronize()
    lm_ms = float(np.mean([lm_t.ms(i) for i in range(args.steps)]))

    # phase 4: per-stage times (one stage at a time, events on the launch stream)
    stage_fns = (("fc", "fc"), ("lm_head", "lm_head"), ("markov", "markov"), ("verify", "verify"))
    if not fp8:
        stage_fns = stage_fns + (("fc_lm_head", "fc_lm"),)
    st_t = LaunchTimer(args.steps * len(stage_fns))
    torch.cuda.synchronize()
    for i in range(args.steps):
        st = slots[i % len(slots)]
        for j, (_, fn) in enumerate(stage_fns):
            st_t.start(i * len(stage_fns) + j, sptr_now)
            check(getattr(st, fn)(), fn)
            st_t.stop(i * len(stage_fns) + j, sptr_now)
    torch.cuda.synchronize()
    stage_us = {name: float(np.mean([st_t.ms(i * len(stage_fns) + j)
                                     for i in range(args.steps)])) * 1e3
                for j, (name, _) in enumerate(stage_fns)}

    # every Markov wait of the timed steps completed: the workspace's error word
    # is sticky until a call with a status word moves it out
    st0 = slots[0]
    st0.status = bufs["status"].data_ptr()
    check(st0.markov(), "drafting (status)")
    torch.cuda.synchronize()
    st0.status = None
    markov_status = int(bufs["status"].item())
    if markov_status != 0:
        raise RuntimeError(f"a bounded wait of the Markov chain gave up (status {markov_status})")

    # algorithmic bytes of each stage (its own inputs and outputs, read or
    # written once); the LM head is the dominant kernel
    rk = w.rank
    if fp8:      # codes + row scales, bf16 hidden states, fp32 logits
        lm_bytes = V * H + V * 4 + B * k * H * es + B * k * V * 4
        fc_bytes = H * w.n_taps * H + H * 4 + w.rows * w.n_taps * H * es + w.rows * H * es
    else:
        lm_bytes = V * H * es + B * k * H * es + B * k * V * 4
        fc_bytes = (H * w.n_taps * H + w.rows * w.n_taps * H + w.rows * H) * es
    markov_bytes = B * k * V * 4 + V * rk * es + B * k * rk * es + B * k * 4
    if sampling:      # x written at j < L_b (the chain generates the draws' noise itself)
        markov_bytes += int(round(float(np.mean(x_positions)) * V * 4))
    conf_bytes = 0 if w.threshold is None else B * k * 4
    verify_b = float(np.mean(verify_bytes)) + B * k * 4 + conf_bytes
    stage_bytes = {"fc": fc_bytes, "lm_head": lm_bytes, "markov": markov_bytes,
                   "verify": verify_b, "fc_lm_head": fc_bytes + lm_bytes}
    stages = {}
    for name, us in stage_us.items():
        gbs = stage_bytes[name] / (us * 1e-6) / 1e9
        stages[name] = {"us": round(us, 2), "bytes": int(stage_bytes[name]),
                        "GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    log("stages: " + ", ".join(f"{n} {v['us']:.1f} us {v['GBs']:.0f} GB/s ({v['frac']:.0%})"
                               for n, v in stages.items()))
    step_bytes = fc_bytes + lm_bytes + markov_bytes + verify_b
    dom_bytes = fc_bytes + lm_bytes if fused else lm_bytes
    achieved = dom_bytes / (lm_ms * 1e-3) / 1e9
    traffic = recorded_traffic(w.name, args.weights, "fc_lm_head_gemm" if fused else "lm_head_gemm")
    log(f"step {ms_step * 1e3:.1f} us ({step_bytes / 1e6:.1f} MB algorithmic = "
        f"{step_bytes / (ms_step * 1e-3) / 1e9:.0f} GB/s); "
        f"{'fc + LM head' if fused else 'LM head'} {lm_ms * 1e3:.1f} us = {achieved:.0f} GB/s")

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one block-step ...")
        cpu = cpu_baseline(w, W, host0,
                           sample=(args.temperature, 0x5EED0000) if sampling else None, fp8=fp8)
        log(f"cpu oracle: {1.0 / cpu['value']:.1f} s per block-step on {cpu['cores']} threads")
        one = cpu_one_thread()
        if one:
            cpu["one_thread"] = one
            log("cpu oracle, one thread: " + ", ".join(
                f"{n} {v['value']:.2f} block-steps/s" for n, v in one.items()))

    out = {
        "metric": "draft+verify block-steps/sec per GPU; HBM GB/s and % roofline",
        "value": 1000.0 / ms_step,
        "unit": "block-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.describe(), "batch": B, "k": k, "hidden": H, "vocab": V,
                   "rank": w.rank, "n_taps": w.n_taps, "threshold": w.threshold,
                   "launch": "hip-graph" if graphs is not None else "eager",
                   "fc_overlap": "none (closed loop)" if args.closed_loop else args.overlap,
                   **({"fc_overlap_auto_us": overlap_choice} if overlap_choice else {}),
                   "loop": "closed" if args.closed_loop else "independent steps",
                   "draft": args.draft,
                   "weights": "fp8-e4m3 codes + fp32 row scales (fc, LM head)" if fp8
                   else ("bf16, fc and LM head in the packed layout (bdr_pack_weight)" if packed
                         else w.dtype),
                   **({"temperature": args.temperature} if sampling else {}),
                   "pool_steps": args.pool,
                   "markov_weights": "one copy" if args.shared_markov else "one copy per slot"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": "LM-head weight-streaming GEMM (dspark_lm_head_fp8)" if fp8
                     else ("fc + LM-head weight-streaming GEMMs in one launch "
                           "(dflash_fuse_fc_lm_head)" if fused
                           else "LM-head weight-streaming GEMM (dspark_lm_head)")
                     + (", packed weights" if packed else ""),
                     "avg_launch_us": lm_ms * 1e3,
                     "algorithmic_bytes_per_launch": dom_bytes},
        "stages": stages,
        "step_algorithmic_bytes": int(step_bytes),
        "step_us": {"mean_back_to_back": ms_step * 1e3, **dist,
                    "note": "rotated: pool slots in turn; cold: 1 GiB read before each step "
                            "(outside its events); warm: slot 0 repeated; per-step events on "
                            "the main stream"},
        "markov_status": markov_status,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
