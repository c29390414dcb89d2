"""Throughput of the LoLA layer hot path on one MI355X.

A step is one lola_prefill_chunk over the 4096-token bf16 GQA workload
(32 query / 8 KV heads, head_dim 128, feature dim 128, window 64, cache 256,
interval 64, batch 1): feature rows, the SRE / top-C / fold interval scan and
the softmax + linear output pass.  Inputs are seeded synthetic tensors already
resident in HBM; every timed step starts from a freshly initialised state.

Also measured: decode (64 sequences with a 4096-token prefilled state, 256
single-token steps), per-kernel times from HIP events recorded between the
library's launches, and the CPU oracle on the host cores as a baseline.

Prints one JSON line.  `--gpus N` with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from sparse_attention_chunkwise_amd import inputs as I  # noqa: E402
from sparse_attention_chunkwise_amd import lola  # noqa: E402

METRIC = "LoLA layer tokens/sec (4K chunkwise prefill; decode) + % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}
PKG = os.path.join(ROOT, "sparse_attention_chunkwise_amd")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def kernel_source_hash():
    """sha256 over the HIP sources and the build script: identifies the kernels a counter run saw."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(PKG, "build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counter runs (already
    scaled by the plain-copy calibration), or None when the kernels changed since those runs."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash() or kernel not in rec.get("kernels", {}):
        return None
    return rec["kernels"][kernel]["bytes"]


# ---------------------------------------------------------------------------
# algorithmic work, from the interval bookkeeping (data independent)
# ---------------------------------------------------------------------------
def interval_plan(layer, T):
    """Per interval of a fresh state: (a, e, |cache| at start, |leaving|, |U|, |folded|)."""
    w, C, L = layer.window, layer.cache_cap, layer.chunk
    cnt, out = 0, []
    for a in range(0, T, L):
        e = min(a + L, T)
        nE = max(0, e - w - max(0, a - w))
        nU = cnt + nE
        keep = min(C, nU)
        out.append((a, e, cnt, nE, nU, nU - keep))
        cnt = keep
    return out


def algorithmic_work(layer, B, T):
    """MACs and bytes each prefill kernel must do by definition (per launch)."""
    D, F, Fh, w, G = layer.head_dim, 2 * layer.feat_half, layer.feat_half, layer.window, layer.group
    chains = B * layer.n_kv_heads
    esize = 2 if layer.io_dtype == "bf16" else 4
    scan = out = 0
    for a, e, cnt, nE, nU, nF in interval_plan(layer, T):
        scan += nU * F * (D + 1) + nF * F * (D + 1)          # SRE (n and d) + fold (H and s)
        for t in range(a, e):
            nwin = min(w, t + 1)
            npend = max(0, t - w - max(0, a - w) + 1)
            out += G * (2 * D * (nwin + cnt) + F * (D + 1) + Fh * D + npend * (F + D + 1))
    prologue = (w + T) * Fh * D
    io = B * T * (2 * layer.n_q_heads + 2 * layer.n_kv_heads) * D * esize  # Q, K, V read, O written
    return {
        "prologue": {"macs": prologue * chains, "bytes": B * T * layer.n_kv_heads * D * esize},
        "scan": {"macs": scan * chains, "bytes": B * T * 2 * layer.n_kv_heads * D * esize},
        "output": {"macs": out * chains, "bytes": io},
        "layer": {"macs": (scan + out + prologue) * chains, "bytes": io},
    }


def decode_bytes(layer, B):
    """Bytes one decode step must move: per chain the state it reads and writes."""
    D, F, w, C = layer.head_dim, 2 * layer.feat_half, layer.window, layer.cache_cap
    esize = 2 if layer.io_dtype == "bf16" else 4
    per_chain = 2 * (F * D + F) * 4 + 2 * C * D * esize + 2 * w * D * esize
    per_chain += (2 * layer.group + 2) * D * esize + 2 * D * esize  # q, out, k, v, slot write
    return per_chain * B * layer.n_kv_heads


def recurrence_bound(layer, B, T, scan_us):
    """Serial intervals per chain and the measured time per interval of the scan."""
    n = len(interval_plan(layer, T))
    return {"intervals": n, "chains": B * layer.n_kv_heads, "us_per_interval": scan_us / n}


# ---------------------------------------------------------------------------
def to_dev(x, layer):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if layer.io_dtype == "bf16" else t


def require_healthy(layer, states, B, what):
    """Exit non-zero if any timed state was marked faulted (a split scan that gave up
    waiting returns early, and its shorter time must not be reported)."""
    for st in states:
        rc = lola.check_state(layer, st, B)
        if rc != 0:
            print(f"bench.py: {what}: a timed state is faulted ({lola.status_string(rc)})", file=sys.stderr)
            sys.exit(3)


def bench_prefill(wl, steps, warmup):
    """Time `steps` prefill launches, each from a fresh state, cold and warm.

    Cold: before every step (outside its events) a 512 MiB buffer is rewritten,
    twice the 256 MB Infinity Cache, so the step reads its inputs from HBM.
    Warm: the same steps back to back with no flush.
    """
    L = wl.layer
    W, Q, K, V = I.make_batch(wl)
    B, T = wl.batch, wl.seq_len
    Wd = torch.from_numpy(W).to("cuda")
    q, k, v = to_dev(Q, L), to_dev(K, L), to_dev(V, L)
    out = torch.empty_like(q)
    ws = torch.empty(lola.workspace_bytes(L, B, T), dtype=torch.uint8, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    states = [lola.init_state(L, B, Wd) for _ in range(2 * steps + warmup)]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(2 * steps)]
    for e4 in ev:  # create the event handles
        for e in e4:
            e.record()
    torch.cuda.synchronize()
    for i in range(warmup):
        lola.prefill(L, states[i], q, k, v, out=out, workspace=ws)
    torch.cuda.synchronize()

    def timed(first, cold):
        t0 = time.perf_counter()
        for i in range(first, first + steps):
            if cold:
                flush.fill_(i & 0xFF)
            lola.prefill_timed(L, states[warmup + i], q, k, v, ev[i], out=out, workspace=ws)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = {"prologue": [], "scan": [], "output": []}
        total = []
        for e4 in ev[first:first + steps]:
            per["prologue"].append(e4[0].elapsed_time(e4[1]))
            per["scan"].append(e4[1].elapsed_time(e4[2]))
            per["output"].append(e4[2].elapsed_time(e4[3]))
            total.append(e4[0].elapsed_time(e4[3]))
        return {
            "ms_per_step": float(np.mean(total)),
            "wall_ms_per_step": 1000.0 * wall / steps,
            "kernel_us": {k: 1000.0 * float(np.mean(v)) for k, v in per.items()},
        }

    cold = timed(0, True)
    warm = timed(steps, False)
    # The headline: lola_prefill_chunk itself, with events only around each call (the
    # timed variant above records events between its three launches, which the step
    # time then includes).  Fresh states again, cold then warm.
    plain_states = [lola.init_state(L, B, Wd) for _ in range(2 * steps)]
    pe = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(2 * steps)]
    for e2 in pe:
        for e in e2:
            e.record()
    torch.cuda.synchronize()

    def plain(first, is_cold):
        for i in range(first, first + steps):
            if is_cold:
                flush.fill_(i & 0xFF)
            pe[i][0].record()
            lola.prefill(L, plain_states[i], q, k, v, out=out, workspace=ws)
            pe[i][1].record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in pe[first:first + steps]]))

    cold["ms_per_step_timed_launches"] = cold["ms_per_step"]
    warm["ms_per_step_timed_launches"] = warm["ms_per_step"]
    cold["ms_per_step"] = plain(0, True)
    warm["ms_per_step"] = plain(steps, False)
    require_healthy(L, states + plain_states, B, "prefill")
    cold["tokens"] = B * T
    cold["warm"] = warm
    return cold


def decode_state(wl, layer):
    """The decode workload's 64 states after their 4096-token prefill (outputs unused)."""
    B, T = wl.batch, wl.seq_len
    Ks, Vs = [], []
    W = None
    for b in range(B):
        Wb, _, K, V, _ = I.make_sequence(wl, b)
        if b == 0:
            W = Wb
        Ks.append(K)
        Vs.append(V)
    Wd = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(W, (layer.n_kv_heads,) + W.shape))).to("cuda")
    k = to_dev(np.stack(Ks), layer)
    v = to_dev(np.stack(Vs), layer)
    del Ks, Vs
    q = torch.zeros((B, T, layer.n_q_heads, layer.head_dim), dtype=k.dtype, device="cuda")
    state = lola.init_state(layer, B, Wd)
    lola.prefill(layer, state, q, k, v)
    del q, k, v
    require_healthy(layer, [state], B, "decode prefill")
    return state


def time_decode(layer, state, B, qd, kd, vd, warmup):
    """Mean per-step time (us) of decode steps from `state`, cold and warm.  Cold: a 512 MiB
    buffer is rewritten before each step, outside its events, so each step reads the
    state from HBM; warm: no flush.  Per-step HIP events on the launch stream."""
    steps = qd.shape[0]
    outd = torch.empty_like(qd[0])
    warm_state = state.clone()
    for s in range(warmup):
        lola.decode(layer, warm_state, qd[s], kd[s], vd[s], out=outd)
    torch.cuda.synchronize()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def timed(st, cold):
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for s in range(steps):
            if cold:
                flush.fill_(s & 0xFF)
            e0[s].record()
            lola.decode(layer, st, qd[s], kd[s], vd[s], out=outd)
            e1[s].record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in zip(e0, e1)])) * 1000.0

    cold_state = state.clone()
    us_cold = timed(cold_state, True)
    us_warm = timed(state, False)
    require_healthy(layer, [cold_state, state, warm_state], B, "decode")
    return us_cold, us_warm


def bench_decode(wl, steps_timed, warmup):
    """64 sequences: 4096-token prefill (untimed) then `steps_timed` decode steps; the same
    with the incremental decode scores (fewer steps) for comparison."""
    L = wl.layer
    B = wl.batch
    state = decode_state(wl, L)
    qd, kd, vd = I.make_decode_steps(wl, steps_timed)
    qd, kd, vd = to_dev(qd, L), to_dev(kd, L), to_dev(vd, L)
    us_cold, us_warm = time_decode(L, state, B, qd, kd, vd, warmup)
    nbytes = decode_bytes(L, B)

    def roof(us, nb=nbytes):
        gbs = nb / (us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "bytes_per_launch": nb, "traffic": measured_traffic("decode")}

    mixed = bench_mixed(wl, state)
    del state
    # incremental decode scores (stored n, d per cached pair): the first step after the
    # prefill recomputes them, so it is one of the untimed warm-up steps
    Li = I.LayerConfig(L.n_q_heads, L.n_kv_heads, L.head_dim, L.feat_half, L.window, L.cache_cap, L.chunk,
                       L.io_dtype, L.softmax_scale, L.policy, 1)
    st_i = decode_state(wl, Li)
    n_i = min(steps_timed, 64)
    lola.decode(Li, st_i, qd[-1], kd[-1], vd[-1])  # the full recomputation, untimed
    ic, iw = time_decode(Li, st_i, B, qd[:n_i], kd[:n_i], vd[:n_i], warmup)
    del st_i
    nb_i = nbytes + B * L.n_kv_heads * 2 * L.cache_cap * (L.head_dim + 1) * 4  # stored n, d read and written
    return {
        "workload": wl.name,
        "value": B / (us_cold * 1e-6),
        "unit": "tokens/s",
        "us_per_step": us_cold,
        "timing": "cold (512 MiB rewritten before each step, outside its events), per-step HIP events",
        "roofline": roof(us_cold),
        "warm": {"value": B / (us_warm * 1e-6), "us_per_step": us_warm, "roofline": roof(us_warm)},
        "incremental_scores": {"us_per_step": ic, "value": B / (ic * 1e-6), "steps": n_i,
                               "warm": {"us_per_step": iw, "value": B / (iw * 1e-6)},
                               "bytes_per_launch": nb_i, "roofline": roof(ic, nb_i)},
        "mixed": mixed,
    }


def bench_mixed(wl, state, steps=8, chunk_tokens=64, n_prefill=8):
    """Continuous batching on the decode workload's states: each lola_prefill_ragged call
    advances n_prefill sequences by a chunk and every other sequence by one token."""
    L = wl.layer
    B = wl.batch
    counts, q, k, v = I.make_mixed_steps(wl, steps + 1, chunk_tokens, n_prefill)
    cd = torch.from_numpy(counts).to("cuda")
    q, k, v = to_dev(q, L), to_dev(k, L), to_dev(v, L)
    out = torch.empty_like(q[0])
    ws = torch.empty(lola.workspace_bytes(L, B, chunk_tokens), dtype=torch.uint8, device="cuda")
    lola.prefill_ragged(L, state, cd[0], q[0], k[0], v[0], out=out, workspace=ws)  # warm-up step
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(1, steps + 1):
        lola.prefill_ragged(L, state, cd[s], q[s], k[s], v[s], out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    require_healthy(L, [state], B, "mixed batch")
    ms = e0.elapsed_time(e1)
    tokens = int(counts[1:].sum())
    return {"workload": f"{wl.name}-mixed-{n_prefill}x{chunk_tokens}+{B - n_prefill}x1",
            "value": tokens / (ms / 1000.0), "unit": "tokens/s", "us_per_step": 1000.0 * ms / steps,
            "tokens_per_step": tokens // steps, "steps": steps}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, wl_dec, dec_seqs=4, dec_steps=16):
    """The fp64 oracle on the host cores: the full 4096-token prefill workload on one thread
    and on all the threads it can use (one per KV-head chain), and a sample of the decode
    workload (dec_seqs of its 64 sequences: their 4096-token prefill in state-only mode,
    untimed, then dec_steps timed decode steps)."""
    import oracle

    nproc = os.cpu_count() or 1
    W, Q, K, V = I.make_batch(wl)
    nthreads = min(nproc, wl.batch * wl.layer.n_kv_heads, 16)
    runs = {}
    for nt in sorted({1, nthreads}):
        orc = oracle.Oracle(wl.layer, wl.batch, W)
        t0 = time.perf_counter()
        orc.run(Q, K, V, nthreads=nt)
        runs[nt] = time.perf_counter() - t0
    # decode sample
    L = wl_dec.layer
    Wd, Qd, Kd, Vd = I.make_batch(wl_dec, batch=dec_seqs)
    qd, kd, vd = I.make_decode_steps(wl_dec, dec_steps, batch=dec_seqs)
    dthreads = min(nproc, dec_seqs * L.n_kv_heads, 16)
    orc = oracle.Oracle(L, dec_seqs, Wd)
    orc.run(None, Kd, Vd, want_out=False, nthreads=dthreads)
    t0 = time.perf_counter()
    for s in range(dec_steps):
        orc.run(qd[s][:, None], kd[s][:, None], vd[s][:, None], nthreads=dthreads)
    dt_dec = time.perf_counter() - t0
    tok = wl.batch * wl.seq_len
    return {"value": tok / runs[nthreads], "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"one full pass of the {wl.seq_len}-token prefill workload (all {wl.layer.n_q_heads} query "
                      f"heads, outputs and state), fp64, {nthreads} threads (one per KV-head chain): "
                      f"{runs[nthreads]:.1f} s",
            "single_thread": {"value": tok / runs[1], "unit": "tokens/s", "cores": 1, "seconds": runs[1]},
            "nproc": nproc, "cpu_model": cpu_model(),
            "decode": {"workload": wl_dec.name, "value": dec_seqs * dec_steps / dt_dec, "unit": "tokens/s",
                       "cores": dthreads, "us_per_step": 1e6 * dt_dec / dec_steps,
                       "sample": f"{dec_seqs} of the {wl_dec.batch} sequences (state-only 4096-token prefill, "
                                 f"untimed), {dec_steps} timed decode steps with outputs, {dthreads} threads"}}


def bench_long(steps=3):
    """The 64K long-context prefill (4 sequences x 65 536 tokens, C 512, L 128): one call per
    fresh state, HIP events between the three launches; one warm-up call first."""
    wl = I.WORKLOADS[5]
    L = wl.layer
    W, Q, K, V = I.make_batch(wl)
    q, k, v = to_dev(Q, L), to_dev(K, L), to_dev(V, L)
    del Q, K, V
    Wd = torch.from_numpy(W).to("cuda")
    out = torch.empty_like(q)
    ws = torch.empty(lola.workspace_bytes(L, wl.batch, wl.seq_len), dtype=torch.uint8, device="cuda")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps + 1)]
    for e4 in ev:  # create the event handles
        for e in e4:
            e.record()
    rows = []
    for i in range(steps + 1):
        st = lola.init_state(L, wl.batch, Wd)
        torch.cuda.synchronize()
        lola.prefill_timed(L, st, q, k, v, ev[i], out=out, workspace=ws)
        torch.cuda.synchronize()
        if lola.check_state(L, st, wl.batch) != 0:
            raise RuntimeError("64K prefill: state marked faulted")
        e = ev[i]
        if i > 0:
            rows.append([e[0].elapsed_time(e[3]), e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]),
                         e[2].elapsed_time(e[3])])
    m = np.mean(np.array(rows), axis=0)
    return {"metric": "LoLA layer tokens/sec (long-context chunkwise prefill)", "workload": wl.name,
            "value": wl.batch * wl.seq_len / (m[0] / 1e3), "unit": "tokens/s", "ms_per_call": m[0],
            "kernel_ms": {"prologue": m[1], "scan": m[2], "output": m[3]},
            "scan_us_per_interval": 1e3 * m[2] / (wl.seq_len // L.chunk), "calls": steps, "data": "synthetic"}


def copy_calibration(nbytes=1 << 30):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE counters."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}), flush=True)


def copy_bandwidth(nbytes=1 << 30, reps=5):
    """Practical HBM ceiling on this GPU: a plain 1 GiB device-to-device copy (torch's copy
    kernel), bytes read + written per second, timed with events over `reps` copies."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1000.0 / reps
    del a, b
    return {"gbs": 2 * nbytes / sec / 1e9, "bytes_per_copy": 2 * nbytes,
            "what": "1 GiB device-to-device copy (read + write), the practical ceiling beside the 8 TB/s peak"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--long-context", action="store_true",
                    help="time only the 64K long-context prefill and print its own JSON line")
    ap.add_argument("--source-hash", action="store_true", help="print the kernel source hash and exit")
    args = ap.parse_args()
    if args.source_hash:
        print(kernel_source_hash())
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the LoLA hot path here runs on one GPU; --gpus must be 1 "
              "(the (sequence, KV head) chains are independent, so they would shard over GPUs with no "
              "collectives)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        copy_calibration()
        return
    if args.long_context:
        print(json.dumps(bench_long()), flush=True)
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.manual_seed(0)
    wl = I.WORKLOADS[3]
    L = wl.layer
    pre = bench_prefill(wl, args.steps, args.warmup)
    work = algorithmic_work(L, wl.batch, wl.seq_len)
    ku = pre["kernel_us"]
    kernels = {}
    for name in ("prologue", "scan", "output"):
        us = ku[name]
        kernels[name] = {"us": us, "tflops": 2 * work[name]["macs"] / (us * 1e-6) / 1e12,
                         "gbs": work[name]["bytes"] / (us * 1e-6) / 1e9}
    dom = max(ku, key=ku.get)
    if dom == "scan":
        # its contraction runs on bf16 MFMAs (hi/lo operand parts): priced at the bf16 dense peak
        roof = {"bound": "mfma", "achieved": kernels["scan"]["tflops"], "peak": PEAK_TFLOPS["bf16"],
                "unit": "TFLOP/s"}
    elif dom == "output":
        roof = {"bound": "mfma", "achieved": kernels["output"]["tflops"], "peak": PEAK_TFLOPS["bf16"],
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kernels[dom]["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom)
    roof["kernel"] = dom
    tok_s = pre["tokens"] / (pre["ms_per_step"] / 1000.0)
    layer_bytes = work["layer"]["bytes"]
    res = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_len, "q_heads": L.n_q_heads,
                   "kv_heads": L.n_kv_heads, "head_dim": L.head_dim, "feat_dim": 2 * L.feat_half,
                   "window": L.window, "cache": L.cache_cap, "chunk": L.chunk},
        "roofline": roof,
        "layer_roofline": {"hbm_bytes": layer_bytes, "t_hbm_us": layer_bytes / HBM_PEAK_GBS / 1e3,
                           "frac_hbm": (layer_bytes / HBM_PEAK_GBS / 1e3) / (pre["ms_per_step"] * 1e3),
                           "macs": work["layer"]["macs"]},
        "kernels": kernels,
        "recurrence": recurrence_bound(L, wl.batch, wl.seq_len, ku["scan"]),
        "wall_ms_per_step": pre["wall_ms_per_step"],
        "timing": "cold (512 MiB rewritten before each step, outside its events); events around each "
                  "lola_prefill_chunk call; per-kernel times from lola_prefill_chunk_timed (events between "
                  "the launches), whose step time is ms_per_step_timed_launches",
        "ms_per_step_timed_launches": pre["ms_per_step_timed_launches"],
        "warm": {"ms_per_step": pre["warm"]["ms_per_step"], "kernel_us": pre["warm"]["kernel_us"],
                 "ms_per_step_timed_launches": pre["warm"]["ms_per_step_timed_launches"],
                 "value": pre["tokens"] / (pre["warm"]["ms_per_step"] / 1000.0)},
    }
    res["hbm_copy"] = copy_bandwidth()
    if not args.no_decode:
        res["decode"] = bench_decode(I.WORKLOADS[4], args.decode_steps, args.warmup)
        for part in (res["decode"]["roofline"], res["decode"]["warm"]["roofline"]):
            part["frac_of_copy"] = part["achieved"] / res["hbm_copy"]["gbs"]
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, I.WORKLOADS[4])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
