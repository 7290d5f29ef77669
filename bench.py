"""Throughput of the SimSD verification hot path on one MI355X.

One step = one pass of the whole path over one batch: the verification
attention (RoPE copy, in-kernel tau mask, split-KV masked GQA attention and
the LSE merge when the prompt is split) followed by the tau-ordered
acceptance walk with its residual draw.  Workload: an SDAR-8B-shaped layer,
batch 32, 32 query / 8 KV heads, head dim 128, prompt 4096, B = gamma = 8,
bf16, acceptance over a 151936-token vocabulary.  Inputs are seeded random
tensors generated on the GPU; two input sets larger than the last-level
cache alternate so no step reads K/V that a previous step left in cache.

Prints ONE JSON line.  `value` is verified candidates per second
(batch * gamma per step).  `roofline` prices the verification call against
the HBM peak using its algorithmic bytes (the K/V stream, each key and value
once, plus the block rows' Q, K and V and the outputs; `kv_frac` gives the
K/V stream alone) and its HIP-event duration on the launch stream, the events taken inside the timed loop on every
--event-stride-th step (an event packet adds a few microseconds to the
step it sits in, so recording them on every step would understate the
throughput); `cpu_baseline` times the fp64 oracle on a bounded sample of the
same workload on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified candidates/sec and achieved HBM TB/s (KV read) at B=8, prompt 4096"
WORKLOAD = "sdar8b_p4096_b8"
VOCAB = 151936
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ("diffusion_lm_speculative_amd/csrc/verify_mfma.hip",
                  "diffusion_lm_speculative_amd/csrc/mfma_common.hpp",
                  "diffusion_lm_speculative_amd/csrc/simsd_common.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_mfma_sdar8b_p4096_b8_traffic.json")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from committed rocprofv3 counters, if the kernel is unchanged since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(t_host, a_host, w, budget_s=12.0):
    """Oracle (fp64 NumPy) over whole sequences until every sequence ran once and ~budget_s of host time passed."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from diffusion_lm_speculative_amd.synth import to_numpy64
    from oracle.acceptance import accept_ref
    from oracle.attention import verify_attn_ref

    cores = len(os.sched_getaffinity(0))  # every core this process may run on
    with threadpool_limits(limits=cores):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        avail = int(t_host["q_blk"].shape[0])
        done = 0
        t0 = time.perf_counter()
        while done < avail or time.perf_counter() - t0 < budget_s:
            b = [done % avail]
            verify_attn_ref(to_numpy64(t_host["q_blk"][b]), to_numpy64(t_host["k_blk"][b]),
                            to_numpy64(t_host["v_blk"][b]), to_numpy64(t_host["k_cache"][b]),
                            to_numpy64(t_host["v_cache"][b]), t_host["prompt_len"][b].numpy(),
                            t_host["tau"][b].numpy(), rope_base=w.rope_base)
            accept_ref(a_host["p"][b].numpy(), a_host["q"][b].numpy(), a_host["draft_tok"][b].numpy(),
                       a_host["tau"][b].numpy(), w.B, 1234, 0)
            done += 1
        dt = time.perf_counter() - t0
    return {"value": done * w.B / dt, "unit": "candidates/s", "cores": int(min(used, cores)), "affinity_cores": cores,
            "kind": "oracle",
            "sample": f"{done} sequence passes cycling over the {avail} sequences of one input set (each: "
                      f"verification attention of {w.Hq} heads x {2 * w.B} rows over {w.P}+{2 * w.B} keys, then the "
                      f"acceptance walk with its residual draw), {dt:.1f} s"}


def call_event_times(torch, sets, stream, n=40):
    """Verify calls timed with events recorded on the stream around each call
    (ms, sorted): the kernel time plus the marker packets' overhead."""
    res = []
    for i in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sets[i % 2]["call"]()
        e1.record(stream)
        e1.synchronize()
        res.append(e0.elapsed_time(e1))
    return sorted(res)


def stream_probe_measure(torch, sd, t, dev, stream, kv_bytes, n=30, warmup=5):
    """The attention kernel's load path alone over the same prompt cache
    (kernel-bound events): the streaming ceiling of that path on this GPU;
    and, beside it, a plain vector-load read of the same bytes."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def timed(fn):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            b.record(stream)
        for _ in range(warmup):
            fn(t["k_cache"], t["v_cache"], sink, stream=stream)
        for a, b in evs:
            fn(t["k_cache"], t["v_cache"], sink, a, b, stream=stream)
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        mean = sum(us) / len(us)
        gbs = kv_bytes / (mean * 1e-6) / 1e9
        return {"us": {"mean": mean, "median": us[len(us) // 2], "min": us[0]}, "bytes": kv_bytes,
                "achieved_gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}

    rec = {"what": "the attention kernel's K/V load path alone (same ring, grid and cache), no attention"}
    rec.update(timed(sd.stream_probe))
    rec["read_probe"] = {"what": "plain 16-byte vector loads of the same K and V bytes into registers "
                                 "(256 workgroups x 512 threads, grid-stride), no LDS"}
    rec["read_probe"].update(timed(sd.read_probe))
    return rec


def mfma_probe_measure(torch, sd, dev, stream, iters=2048, n=5):
    """The bf16 matrix cores alone (simsd_mfma_probe: independent 32x32x16
    MFMAs on registers, kernel-bound events) at 1, 2 and 4 waves per SIMD:
    the compute-side ceiling the MFMA kernels are compared with."""
    res = {"what": "independent v_mfma_f32_32x32x16_bf16 on registers, no memory traffic in the loop",
           "iters": iters, "peak_tflops_published": MFMA_BF16_PEAK_TFLOPS}
    best = 0.0
    for waves_per_simd in (1, 2, 4):
        wgs = 256 * waves_per_simd
        sink = torch.zeros(wgs * sd.api.MFMA_PROBE_THREADS, dtype=torch.float32, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            b.record(stream)
        sd.mfma_probe(wgs, 16, sink, stream=stream)
        for a, b in evs:
            sd.mfma_probe(wgs, iters, sink, a, b, stream=stream)
        torch.cuda.synchronize()
        us = min(a.elapsed_time(b) * 1e3 for a, b in evs)
        flops = wgs * 4 * iters * sd.api.MFMA_PROBE_FLOPS_PER_ROUND
        tflops = flops / (us * 1e-6) / 1e12
        best = max(best, tflops)
        res[f"waves_per_simd_{waves_per_simd}"] = {"us_min": us, "tflops": tflops}
    res["tflops_best"] = best
    res["frac_of_published_peak"] = best / MFMA_BF16_PEAK_TFLOPS
    return res


def ablation_measure(torch, sd, w, sets, dev, stream, n=20):
    """The no-RoPE-copy ablation on the bench workload: the same verify call
    with the mask slots at their own sequential positions (rope_mode =
    SIMSD_ROPE_SEQUENTIAL) against the RoPE copy, kernel-bound events,
    calls interleaved over both input sets."""
    calls = {}
    for mode_name, mode in (("rope_copy", sd.ROPE_COPY), ("rope_sequential", sd.ROPE_SEQUENTIAL)):
        per_set = []
        for s in sets:
            t = s["t"]
            out = torch.empty_like(t["q_blk"])
            desc = sd.make_desc(t["q_blk"], t["k_blk"], t["k_cache"], rope_base=w.rope_base, rope_mode=mode)
            ws = torch.empty(max(sd.verify_workspace_bytes(desc), 256), dtype=torch.uint8, device=dev)
            per_set.append(sd.bind_verify(t["q_blk"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["tau"],
                                          t["prompt_len"], None, out=out, workspace=ws, stream=stream,
                                          rope_base=w.rope_base, rope_mode=mode))
        calls[mode_name] = per_set
    evs = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
           for k in calls}
    for k in evs:
        for a, b in evs[k]:
            a.record(stream)
            b.record(stream)
    for i in range(4):
        for k in calls:
            calls[k][i % 2]()
    for i in range(n):
        for k in calls:
            a, b = evs[k][i]
            calls[k][i % 2].timed(a, b)
    torch.cuda.synchronize()
    res = {"what": "verify call with the mask slots at sequential positions (no RoPE copy) against the RoPE copy"}
    for k in calls:
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs[k])
        res[k] = {"us": {"mean": sum(us) / len(us), "median": us[len(us) // 2]}}
    return res


def c5_measure(torch, sd, synth, dev, stream, steps=20, warmup=3):
    """The verification-plus-acceptance workload at batch 64 (32/8 heads,
    head dim 128, prompts uniform in [2048, 16384], B = gamma = 16,
    accept_prefix over [64][16][151936]): one step is a verify call and an
    accept_prefix call with its residual draw, two input sets alternating.
    Kernel-bound events on the verify call (attention kernel start to merge
    end), an event after the acceptance."""
    w = synth.WORKLOADS["sdar8b_var16k_b16_accept"]
    gamma = w.gamma
    sets = []
    for i in range(2):
        t = synth.make_verify_inputs(w, 5005 + 100 * i, device=dev)
        a = synth.make_accept_inputs(w.NB, w.B, w.vocab, seed=6006 + 100 * i, device=dev)
        out = torch.empty_like(t["q_blk"])
        desc = sd.make_desc(t["q_blk"], t["k_blk"], t["k_cache"], rope_base=w.rope_base)
        ws = torch.empty(max(sd.verify_workspace_bytes(desc), 256), dtype=torch.uint8, device=dev)
        st = torch.empty((w.NB,), dtype=torch.int32, device=dev)
        call = sd.bind_verify(t["q_blk"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["tau"],
                              t["prompt_len"], None, out=out, status=st, workspace=ws, stream=stream,
                              rope_base=w.rope_base)
        n_acc = torch.empty((w.NB,), dtype=torch.int32, device=dev)
        nxt = torch.empty_like(n_acc)
        ast = torch.empty_like(n_acc)
        aws = torch.empty(max(sd.accept_workspace_bytes(w.NB, w.B, w.vocab), 256), dtype=torch.uint8, device=dev)
        acc = sd.bind_accept(a["p"], a["q"], a["draft_tok"], a["tau"], gamma, n_accepted=n_acc, next_token=nxt,
                             status=ast, workspace=aws, stream=stream)
        sets.append(dict(t=t, call=call, acc=acc, st=st, ast=ast, kv=w.kv_bytes(t["prompt_len"])))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        e[1].record(stream)
    for i in range(warmup):
        sets[i % 2]["call"]()
        sets[i % 2]["acc"](4321, i)
    torch.cuda.synchronize()
    for k, s_ in enumerate(sets):
        if int(s_["st"].abs().sum()) or int(s_["ast"].abs().sum()):
            raise RuntimeError(f"batch-64 input set {k}: device status flags set")
    t0 = time.perf_counter()
    for i in range(steps):
        s_ = sets[i % 2]
        s_["call"].timed(evs[i][0], evs[i][1])
        s_["acc"](4321, i)
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    v_us = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    a_us = [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
    kv = [sets[i % 2]["kv"] / (v_us[i] * 1e-6) / 1e9 for i in range(steps)]
    us_step = wall * 1e6 / steps
    return {"workload": w.name, "batch": w.NB, "B": w.B, "gamma": gamma, "vocab": w.vocab,
            "us_per_step": us_step, "candidates_per_s": w.NB * gamma / (us_step * 1e-6),
            "verify_us": {"mean": sum(v_us) / steps, "median": sorted(v_us)[steps // 2]},
            "accept_us": {"mean": sum(a_us) / steps, "median": sorted(a_us)[steps // 2]},
            "kv_gbs_mean": sum(kv) / steps, "kv_frac": sum(kv) / steps / HBM_PEAK_GBS,
            "kv_bytes_sets": [s_["kv"] for s_ in sets]}


def copy_calibration(torch, dev, mib, steps, warmup):
    """A plain copy of known size: each launch reads and writes mib MiB once."""
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / max(steps, 1)
    print(json.dumps({"copy_mib": mib, "bytes_read": n * 4, "bytes_written": n * 4, "us_per_copy": us,
                      "gbs_read_plus_write": 2 * n * 4 / (us * 1e-6) / 1e9}), flush=True)


def kernel_only(torch, sd, synth, dev, name, calls):
    """Repeated calls of one kernel and nothing else, for counter runs: a
    verification workload by name (one input set), or "projection" (the QKV
    projection at 512 rows x hidden 4096 -> 6144)."""
    if name == "projection":
        x, wt = synth.make_linear_inputs(512, 4096, 6144, seed=3, device=dev)
        y = torch.empty((512, 6144), dtype=torch.bfloat16, device=dev)
        call = sd.bind_linear(x, wt, y)
    else:
        w = synth.WORKLOADS[name]
        t = synth.make_verify_inputs(w, 5, device=dev)
        out = torch.empty_like(t["q_blk"])
        desc = sd.make_desc(t["q_blk"], t["k_blk"], t["k_cache"], rope_base=w.rope_base)
        ws = torch.empty(max(sd.verify_workspace_bytes(desc), 256), dtype=torch.uint8, device=dev)
        call = sd.bind_verify(t["q_blk"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["tau"],
                              t["prompt_len"], None, out=out, workspace=ws, rope_base=w.rope_base)
    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    print(json.dumps({"kernel_only": name, "calls": calls}), flush=True)


def coupled_measure(torch, sd, synth, dev, stream, steps, warmup):
    """Coupled-noise acceptance over full vocabulary rows, timed on its own.

    Workload: batch 64, B = gamma = 16, V = 151936, p = softmax of N(0, 2)
    logits, Exp(1) noise.  Drafts hold the target token (argmax of p/E,
    taken here with plain torch ops) for the first m stages of each sequence,
    m uniform in 0..gamma, so the walk's lengths spread; the kernel reads
    every walked row whatever the outcome.  Algorithmic bytes per call:
    batch * gamma rows of p and E, V * 4 bytes each.
    """
    w = synth.WORKLOADS["sdar8b_var16k_b16_accept"]
    NB, B, gamma, V = w.NB, w.B, w.gamma, w.vocab
    sets = []
    for i in range(2):  # two sets of 1.245 GB: larger than the last-level cache
        a = synth.make_accept_inputs(NB, B, V, seed=3003 + 100 * i, device=dev)
        del a["q"]
        e = synth.make_noise_exp(NB, B, V, seed=3004 + 100 * i, device=dev)
        target = torch.argmax(a["p"] / e, dim=-1).to(torch.int32)
        g = torch.Generator(device=dev)
        g.manual_seed(3005 + 100 * i)
        m = torch.randint(0, gamma + 1, (NB, 1), generator=g, device=dev, dtype=torch.int32)
        draft = torch.where(a["tau"] <= m, target, a["draft_tok"]).contiguous()
        n = torch.empty((NB,), dtype=torch.int32, device=dev)
        nx = torch.empty_like(n)
        st = torch.empty_like(n)
        ws = torch.empty(sd.accept_coupled_workspace_bytes(NB, B, V), dtype=torch.uint8, device=dev)
        call = sd.bind_accept_coupled(a["p"], e, draft, a["tau"], gamma, n_accepted=n, next_token=nx, status=st,
                                      workspace=ws, stream=stream)
        sets.append(dict(call=call, n=n, st=st, m=m))
    torch.cuda.synchronize()
    for s in sets:
        s["call"]()
    torch.cuda.synchronize()
    if any(int(s["st"].abs().sum()) for s in sets):
        raise RuntimeError("coupled acceptance: device status flags set")
    mean_n = sum(float(s["n"].float().mean()) for s in sets) / len(sets)
    for i in range(warmup):
        sets[i % 2]["call"]()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        sets[i % 2]["call"]()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    avg = sum(ms) / len(ms)
    nbytes = NB * gamma * V * 4 * 2
    gbs = nbytes / (avg * 1e-3) / 1e9
    return {"workload": "batch 64, B = gamma = 16, V = 151936, fp32 p and Exp(1) noise",
            "us": {"mean": avg * 1e3, "median": ms[len(ms) // 2] * 1e3}, "mean_n_accepted": mean_n,
            "algorithmic_bytes": nbytes, "achieved_gbs": gbs, "frac": gbs / HBM_PEAK_GBS}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def projection_measure(torch, sd, synth, dev, stream, steps, warmup):
    """The projections around the attention at the same layer shape (32
    sequences x 16 block rows = 512 rows, hidden 4096, 32 query / 8 KV heads
    of 128): the fused QKV projection (4096 -> 6144 channels) and the output
    projection (4096 -> 4096).  Eight weight sets rotate (400 MB, more than
    the last-level cache), as the layers of a model would; each timed block
    is 8 back-to-back calls between two events on the launch stream.
    """
    M, H, Hq, Hkv, d = 512, 4096, 32, 8, 128
    nsets = 8
    res = {}

    def timed(calls):
        for i in range(max(warmup, nsets)):
            calls[i % nsets]()
        per_call = []
        for _ in range(max(steps // nsets, 4)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for c in calls:
                c()
            e1.record(stream)
            e1.synchronize()
            per_call.append(e0.elapsed_time(e1) / nsets)
        per_call.sort()
        return sum(per_call) / len(per_call) * 1e3, per_call[len(per_call) // 2] * 1e3

    for name, N, K in (("qkv_proj", (Hq + 2 * Hkv) * d, H), ("o_proj", H, Hq * d)):
        calls = []
        lib_calls = []  # the vendor GEMM (hipBLASLt through torch.mm) on the same operands, for reference
        for i in range(nsets):
            x, w = synth.make_linear_inputs(M, K, N, seed=4000 + 10 * i + (name == "o_proj"), device=dev)
            y_ref = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            lib_calls.append(lambda x=x, w=w, y=y_ref: torch.mm(x, w.t(), out=y))
            if name == "qkv_proj":
                q = torch.empty((32, 16, Hq, d), dtype=torch.bfloat16, device=dev)
                k = torch.empty((32, 16, Hkv, d), dtype=torch.bfloat16, device=dev)
                v = torch.empty_like(k)
                calls.append(sd.bind_qkv_proj(x.view(32, 16, H), w, Hq, Hkv, d, q, k, v, stream=stream))
            else:
                out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                calls.append(sd.bind_linear(x, w, out, stream=stream))
        torch.cuda.synchronize()
        us, med = timed(calls)
        lib_us, lib_med = timed(lib_calls)
        flops = 2.0 * M * N * K
        tflops = flops / (us * 1e-6) / 1e12
        res[name] = {"M": M, "N": N, "K": K, "us": {"mean": us, "median": med},
                     "tflops": tflops, "frac_mfma_bf16": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "weight_gbs": N * K * 2 / (us * 1e-6) / 1e9,
                     "library_reference": {"what": "torch.mm (hipBLASLt), y = x W^T on the same operands, "
                                                   "same timing; context only, not on the path",
                                           "us": {"mean": lib_us, "median": lib_med},
                                           "tflops": flops / (lib_us * 1e-6) / 1e12}}
    return res


def commit_measure(torch, sd, w, sets, dev, stream, steps):
    """The commit step of the headline workload: simsd_next_round (the next
    round's labels and tokens), simsd_commit of one round (the accept outputs
    of an input set) and simsd_append_kv of the finished
    blocks (every block counted as finished: 32 sequences x 8 data rows x 8
    KV heads of K and V, keys rotated) into a cache with room for the 8 calls
    of a timed block (the lengths are reset between blocks, outside the
    events).  Mean per call over blocks of 8 calls between two events."""
    NB, B = w.NB, w.B
    s = sets[0]
    committed = torch.zeros(NB, dtype=torch.int64, device=dev)
    block_tok = torch.full((NB, B), -1, dtype=torch.int32, device=dev)
    p_max = w.P + 8 * B
    kc = torch.zeros((NB, w.Hkv, p_max, w.d), dtype=w.dtype, device=dev)
    vc = torch.zeros_like(kc)
    plen = torch.full((NB,), w.P, dtype=torch.int32, device=dev)
    rank = torch.randint(0, B, (NB, B), dtype=torch.int32, device=dev)
    tau_next = torch.empty((NB, B), dtype=torch.int32, device=dev)
    tok_next = torch.empty_like(tau_next)
    calls = {
        "next_round": sd.bind_next_round(committed, block_tok, s["a"]["draft_tok"], rank, tau_next, tok_next,
                                         stream=stream),
        "commit": sd.bind_commit(s["a"]["tau"], s["a"]["draft_tok"], s["n_acc"], s["nxt"], committed, block_tok,
                                 stream=stream),
        "append_kv": sd.bind_append_kv(s["t"]["k_blk"], s["t"]["v_blk"], kc, vc, plen, rope_base=w.rope_base,
                                       stream=stream),
    }
    res = {}
    for name, call in calls.items():
        times = []
        for it in range(max(steps // 8, 4) + 1):
            plen.fill_(w.P)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(8):
                call()
            e1.record(stream)
            e1.synchronize()
            if it:  # the first block is the warmup
                times.append(e0.elapsed_time(e1) / 8 * 1e3)
        res[name + "_us"] = sum(times) / len(times)
    # K and V rows read from the block and written to the cache
    res["append_bytes_moved"] = 4 * NB * B * w.Hkv * w.d * (2 if w.dtype == torch.bfloat16 else 4)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--kernel-only", default=None,
                    help="only repeat one kernel --steps times (a verification workload name, or "
                         "'projection'), for hardware-counter runs; prints no bench line")
    ap.add_argument("--event-stride", type=int, default=5,
                    help="time verify and accept on every N-th timed step (each event packet adds a few "
                         "microseconds to its step); N odd, so that the two alternating input sets are sampled "
                         "equally")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the host oracle timing")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only run the streaming probe over the bench workload's prompt cache --steps times "
                         "(for kernel-trace runs); prints its JSON")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the bench, time a plain device-to-device copy of MIB MiB (the known-size "
                         "reference that HBM byte counters are scaled by)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (this path has no multi-GPU "
              "mode: each GPU would run its own share of sequences independently)", file=sys.stderr)
        sys.exit(2)

    import torch

    import diffusion_lm_speculative_amd as sd
    from diffusion_lm_speculative_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(torch, dev, args.copy_calibration, args.steps, args.warmup)
        return
    if args.kernel_only:
        kernel_only(torch, sd, synth, dev, args.kernel_only, args.steps)
        return
    w = synth.WORKLOADS[WORKLOAD]
    gamma = w.B
    stream = torch.cuda.current_stream()
    if args.stream_probe:
        t = synth.make_verify_inputs(w, 1002, device=dev)
        print(json.dumps({"stream_probe": stream_probe_measure(torch, sd, t, dev, stream, w.kv_bytes(),
                                                               n=args.steps)}), flush=True)
        return

    # Two input sets (each ~537 MB of K/V, together > the 256 MB last-level cache).
    sets = []
    for i in range(2):
        t = synth.make_verify_inputs(w, 1002 + 100 * i, device=dev)
        a = synth.make_accept_inputs(w.NB, w.B, VOCAB, seed=2002 + 100 * i, device=dev)
        out = torch.empty_like(t["q_blk"])
        lse = torch.empty((w.NB, 2 * w.B, w.Hq), dtype=torch.float32, device=dev)
        st = torch.empty((w.NB,), dtype=torch.int32, device=dev)
        desc = sd.make_desc(t["q_blk"], t["k_blk"], t["k_cache"], rope_base=w.rope_base)
        ws_bytes = sd.verify_workspace_bytes(desc)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        call = sd.bind_verify(t["q_blk"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["tau"],
                              t["prompt_len"], None, out=out, lse=lse, status=st, workspace=ws, stream=stream,
                              rope_base=w.rope_base)
        n_acc = torch.empty((w.NB,), dtype=torch.int32, device=dev)
        nxt = torch.empty((w.NB,), dtype=torch.int32, device=dev)
        ast = torch.empty((w.NB,), dtype=torch.int32, device=dev)
        aws = torch.empty(max(sd.accept_workspace_bytes(w.NB, w.B, VOCAB), 256), dtype=torch.uint8, device=dev)

        bound = sd.bind_accept(a["p"], a["q"], a["draft_tok"], a["tau"], gamma, n_accepted=n_acc, next_token=nxt,
                               status=ast, workspace=aws, stream=stream)

        def accept(bound=bound, i=i):
            bound(1234, i)

        sets.append(dict(t=t, a=a, call=call, accept=accept, out=out, lse=lse, st=st, ws=ws, n_acc=n_acc,
                         nxt=nxt, ast=ast, aws=aws))
    torch.cuda.synchronize()

    # On the event steps the verify call takes its two events bound to its own
    # kernel (start and end of the attention kernel, hipExtLaunchKernel):
    # events recorded around the call add marker packets whose few
    # microseconds are not the kernel's.  The acceptance is timed from the
    # end of that kernel to an event recorded after the acceptance call.
    def step(i, ev=None):
        s = sets[i % 2]
        if ev is not None:
            s["call"].timed(ev[0], ev[1])
        else:
            s["call"]()
        s["accept"]()
        if ev is not None:
            ev[2].record(stream)

    # one validation pass over each input set, then the untimed warmup
    for i in range(len(sets)):
        step(i)
    torch.cuda.synchronize()
    for k, s in enumerate(sets):
        if int(s["st"].abs().sum()) or int(s["ast"].abs().sum()):
            raise RuntimeError(f"input set {k}: device status flags set: verify {s['st'].tolist()} "
                               f"accept {s['ast'].tolist()}")
    for i in range(args.warmup):
        step(i)

    stride = max(1, args.event_stride)
    if stride % 2 == 0:
        stride += 1  # an even stride would time only one of the two alternating input sets
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(0, args.steps, stride)]
    for e in evs:  # HIP creates an event at its first record; the kernel-bound ones then re-record it
        e[0].record(stream)
        e[1].record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i // stride] if i % stride == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    verify_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    accept_ms = sorted(e[1].elapsed_time(e[2]) for e in evs)
    v_avg = sum(verify_ms) / len(verify_ms)
    a_avg = sum(accept_ms) / len(accept_ms)
    ms_per_step = wall * 1e3 / args.steps
    kv_bytes = w.kv_bytes()
    # bytes the call must move besides the K/V stream: the block rows' Q, K
    # and V, the output rows and lse
    esz = 2
    q_bytes = w.NB * 2 * w.B * w.Hq * w.d * esz
    alg_parts = {"kv_cache": kv_bytes, "q_blk": q_bytes, "kv_blk": 2 * w.NB * 2 * w.B * w.Hkv * w.d * esz,
                 "out": q_bytes, "lse": w.NB * 2 * w.B * w.Hq * 4}
    alg_bytes = sum(alg_parts.values())
    achieved_gbs = alg_bytes / (v_avg * 1e-3) / 1e9
    kv_gbs = kv_bytes / (v_avg * 1e-3) / 1e9
    desc = sd.make_desc(sets[0]["t"]["q_blk"], sets[0]["t"]["k_blk"], sets[0]["t"]["k_cache"], rope_base=w.rope_base)
    traffic = measured_traffic()

    call_ms = call_event_times(torch, sets, stream)
    probe = stream_probe_measure(torch, sd, sets[0]["t"], dev, stream, kv_bytes)
    coupled = coupled_measure(torch, sd, synth, dev, stream, args.steps, args.warmup)
    projections = projection_measure(torch, sd, synth, dev, stream, args.steps, args.warmup)
    commit_times = commit_measure(torch, sd, w, sets, dev, stream, args.steps)
    mfma_ceiling = mfma_probe_measure(torch, sd, dev, stream)
    ablation = ablation_measure(torch, sd, w, sets, dev, stream)
    nb = w.NB
    t_host = {k: v[:nb].cpu() for k, v in sets[0]["t"].items()}
    a_host = {k: v[:nb].cpu() for k, v in sets[0]["a"].items()}
    c5 = c5_measure(torch, sd, synth, dev, stream)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(t_host, a_host, w)

    rec = {
        "metric": METRIC,
        "value": w.NB * gamma / (ms_per_step * 1e-3),
        "unit": "candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.25) q/k/v/cache, softmax(N(0,2)) p/q, random tau permutations)",
        "config": {"workload": WORKLOAD, "batch": w.NB, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "prompt_len": w.P, "B": w.B, "gamma": gamma, "vocab": VOCAB, "kv_chunk": 0},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "verify_mfma_kernel (+ lse merge when split)", "algorithmic_bytes": alg_bytes,
                     "algorithmic_parts": alg_parts, "kv_frac": kv_gbs / HBM_PEAK_GBS},
        "kv_tb_per_s": kv_gbs / 1e3,
        "verify_us": {"mean": v_avg * 1e3, "median": verify_ms[len(verify_ms) // 2] * 1e3,
                      "p90": verify_ms[int(len(verify_ms) * 0.9)] * 1e3, "samples": len(verify_ms),
                      "event_stride": stride, "events": "bound to the attention kernel's own dispatch"},
        "verify_call_us": {"mean": sum(call_ms) / len(call_ms) * 1e3, "median": call_ms[len(call_ms) // 2] * 1e3,
                           "samples": len(call_ms), "events": "recorded on the stream around each call"},
        "stream_probe": probe,
        "accept_us": {"mean": a_avg * 1e3, "median": accept_ms[len(accept_ms) // 2] * 1e3},
        "workspace_bytes": sd.verify_workspace_bytes(desc),
        "cpu_baseline": cpu,
        "accept_coupled": coupled,
        "projections": projections,
        "commit_step": commit_times,
        "mfma_probe": mfma_ceiling,
        "verify_accept_batch64": c5,
        "ablation_no_rope_copy": ablation,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
