"""Benchmark of the HeadKV decode-time path on one MI355X.

One benchmark step = one pass of the whole path over one batch: classification
and initial layout (hkv_classify), then every decode step t = P .. N-1 as one
fused launch (hkv_decode_step: append + attention with the eviction-score
side-output + Stratified Token Eviction) over all layers x sequences x heads
(layer-folded launch).  Inputs are synthetic, seeded, generated on the device
before timing and resident in HBM.

Default workload: LlamaGen-XL-shaped, bf16, 36 layers x 16 sequences x 20 heads,
head_dim 64, N = 696, P = 184, rho = 1/6 (512 decode steps).

Prints ONE JSON line.  value = generated tokens per second = batch * decode
steps / step time.  The roofline block is for the dominant kernel (the fused
decode step): algorithmic bytes per launch / mean launch time, from HIP events
recorded on the launch stream around each timed generation's decode loop and
divided by its launches.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "compressed decode-attn tokens/s at rho=1/6; achieved HBM GB/s as % of peak"
KERNEL_SOURCES = ("kv_cache_compression_hkv_amd/csrc/hkv_kernels.hip",
                  "kv_cache_compression_hkv_amd/csrc/hkv_device.h")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hkv_decode_step_llamagen_xl_counters.json")


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\])*"|//[^\n]*|/\*.*?\*/', re.S)


def kernel_hash() -> str:
    """Hash of the kernel sources' code: comments and whitespace do not count,
    so a recorded counter run stays valid until the code itself changes."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        code = _CODE_TOKENS.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- bytes model
def step_bytes(labels, budgets, w):
    """Algorithmic bytes of every fused decode launch of one generation.

    Per stream and step, with c the slots holding a token after the append and
    e the element size: K and V rows 2*d*e*c, query in and output out 2*d*e,
    append write 2*d*e + 8 (row, position, score reset for Global streams) and
    33 bytes of per-stream metadata (label, extent, capacity, budget, base, free
    count; extent written back).  A Global stream at an eviction step also reads
    its W-query window ((W-1)*d*e beyond the current query) and the positions of
    its c slots (4*c), and writes its free list, the freed positions and the free
    count (8*M + 4).
    """
    import numpy as np
    d, e, M, P, T, W = w.head_dim, w.elem_bytes, w.evict_m, w.P, w.steps, w.w_obs
    row = d * e
    base_bytes = lambda c: 2 * row * c + 2 * row + 2 * row + 8 + 33
    out = np.zeros(T)
    glob, local = {}, {}
    for lab, B in zip(labels.tolist(), budgets.tolist()):
        if lab == 2:                       # full cache
            out += base_bytes(np.arange(P + 1, P + T + 1))
            continue
        if lab == 0:                       # local ring of B slots
            local[B] = local.get(B, 0) + 1
            continue
        glob[B] = glob.get(B, 0) + 1
    for B, n in local.items():
        out += n * base_bytes(np.minimum(np.arange(P + 1, P + T + 1), B))
    for B, n in glob.items():
        cnt = min(P, B)
        traj = np.zeros(T)
        for i in range(T):
            c = cnt + 1
            b = base_bytes(c)
            if c == B + M:
                b += (W - 1) * row + 4 * c + 8 * M + 4
                cnt = B
            else:
                cnt = c
            traj[i] = b
        out += n * traj
    return out


def attn_bytes(labels, budgets, w):
    """Algorithmic bytes of every attention launch (hkv_decode_attn) of one
    generation run as separate calls: per stream and step the K and V rows of
    its c slots (2*d*e*c), query in and output out (2*d*e), the query-statistics
    ring entry written (16) and 29 bytes of metadata read.  The append before it
    and the eviction after it are separate launches."""
    import numpy as np
    d, e, M, P, T = w.head_dim, w.elem_bytes, w.evict_m, w.P, w.steps
    row = d * e
    one = lambda c: 2 * row * c + 2 * row + 16 + 29
    out = np.zeros(T)
    for lab, B in zip(labels.tolist(), budgets.tolist()):
        steps = np.arange(P + 1, P + T + 1)
        if lab == 2:
            out += one(steps)
        elif lab == 0:
            out += one(np.minimum(steps, B))
        else:
            cnt = min(P, B)
            for i in range(T):
                c = cnt + 1
                out[i] += one(c)
                cnt = B if c == B + M else c
    return out


# ---------------------------------------------------------------- CPU baseline
def _oracle_worker(args):
    """Runs the oracle on a list of (layer, sequence) groups, one after another;
    only run_group is timed (each group's inputs are generated just before)."""
    name, groups, seed = args
    from hkv_inputs.configs import WORKLOADS
    from hkv_inputs import gen
    import oracle.hkv_oracle as O
    w = WORKLOADS[name]
    busy = 0.0
    for (l, b) in groups:
        kb, vb, qb = gen.group_inputs(w, seed, l, b)
        K, V, Q = gen.decode(kb, w.dtype), gen.decode(vb, w.dtype), gen.decode(qb, w.dtype)
        t0 = time.perf_counter()
        O.run_group(w, K, V, Q)
        busy += time.perf_counter() - t0
    return busy, len(groups)


def cpu_baseline(w, seed: int, max_groups_per_core: int = 36):
    """The oracle on the host cores: every (layer, sequence) group of the
    workload, up to `max_groups_per_core` per core, spread over one process per
    core.  Throughput = generated tokens of the groups run / the busiest
    process's oracle time, where a token is one sequence through all layers."""
    import multiprocessing as mp
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    n = min(w.layers * w.batch, cores * max_groups_per_core)
    groups = [(g % w.layers, g // w.layers) for g in range(n)]
    chunks = [(w.name, groups[i::cores], seed) for i in range(cores)]
    ctx = mp.get_context("spawn")
    env = dict(OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        with ctx.Pool(cores) as pool:
            res = pool.map(_oracle_worker, chunks)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    wall = max(r[0] for r in res)
    n_groups = sum(r[1] for r in res)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    tokens = n_groups * w.steps / w.layers
    whole = "the whole workload" if n_groups == w.layers * w.batch else "a sample"
    return {"value": tokens / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "wall_s": round(wall, 2),
            "sample": f"{n_groups} of {w.layers * w.batch} (layer, sequence) groups of {w.name} "
                      f"({whole}), every decode step, numpy fp64, one process per core, "
                      f"{wall:.1f} s of oracle time on the busiest core"}


# ---------------------------------------------------------------- GPU run
class Generation:
    def __init__(self, w, inputs, hk):
        import torch
        self.w, self.hk = w, hk
        self.K, self.V, self.Q = inputs
        self.cfg = hk.config_from_workload(w)
        self.cache = hk.HkvCache(self.cfg)
        self.out = torch.empty((w.S, w.head_dim), dtype=self.K.dtype, device=self.K.device)
        d, eb = w.head_dim, w.elem_bytes
        self.kp = [self.K.data_ptr() + t * d * eb for t in range(w.N)]
        self.vp = [self.V.data_ptr() + t * d * eb for t in range(w.N)]
        # window of the W newest queries (positions t-W+1 .. t) for step t
        self.qw = [self.Q.data_ptr() + (t - w.w_obs + 1 - (w.P - w.w_obs)) * d * eb
                   for t in range(w.N)]

    def run(self, stream, events=None, capture=None, separate=False):
        """One generation; `events` = (start, end) recorded around the decode loop;
        `capture` ([steps, S, d], untimed use only) receives every step's output;
        `separate`: each decode step as its three calls (hkv_append,
        hkv_decode_attn, hkv_ste_evict), which give the fused step's bits."""
        w, hk, st = self.w, self.hk, self.cache.state
        d, eb = w.head_dim, w.elem_bytes
        hk.hkv_classify(self.cfg, st, self.K, self.V, w.N * d, self.Q, w.q_rows * d, stream)
        if events is not None:
            events[0].record(stream)
        for t in range(w.P, w.N):
            if separate:
                q_cur = self.qw[t] + (w.w_obs - 1) * d * eb      # the query of position t
                hk.hkv_append(self.cfg, st, t, self.kp[t], self.vp[t], w.N * d, 0, w.S, stream)
                hk.hkv_decode_attn(self.cfg, st, t, q_cur, w.q_rows * d, self.out, d, 0, w.S,
                                   stream)
                hk.hkv_ste_evict(self.cfg, st, t, self.qw[t], w.q_rows * d, None, 0, w.S,
                                 stream)
            else:
                hk.hkv_decode_step(self.cfg, st, t, self.kp[t], self.vp[t], w.N * d,
                                   self.qw[t], w.q_rows * d, self.out, d, None, 0, w.S, stream)
            if capture is not None:
                capture[t - w.P].copy_(self.out)
        if events is not None:
            events[1].record(stream)


# decode steps per captured graph of the per-layer loop: a graph of a whole
# generation holds up to 1.4e5 launches (Lumina-mGPT, split step), and the HIP
# runtime ended the process on the host while instantiating one of that size
GRAPH_STEPS = 64


def decode_per_layer(gen_obj, stream, n_split=0, t_begin=None, t_end=None):
    """The decode loop as a model runs it: at every step one launch per layer,
    each over that layer's batch x heads streams (n_split > 0: the split decode
    step, two kernels per layer).  Steps t_begin .. t_end-1 (default all)."""
    w, hk, st = gen_obj.w, gen_obj.hk, gen_obj.cache.state
    d, per = w.head_dim, w.batch * w.heads
    t_begin = w.P if t_begin is None else t_begin
    t_end = w.N if t_end is None else t_end
    for t in range(t_begin, t_end):
        for l in range(w.layers):
            if n_split:
                hk.hkv_decode_step_split(gen_obj.cfg, st, t, gen_obj.kp[t], gen_obj.vp[t],
                                         w.N * d, gen_obj.qw[t], w.q_rows * d, gen_obj.out, d,
                                         None, l * per, per, n_split, stream)
            else:
                hk.hkv_decode_step(gen_obj.cfg, st, t, gen_obj.kp[t], gen_obj.vp[t], w.N * d,
                                   gen_obj.qw[t], w.q_rows * d, gen_obj.out, d, None, l * per,
                                   per, stream)


def time_per_layer(gen_obj, steps, splits=(2, 4, 8)):
    """Per-layer decode loop, launched eagerly and replayed as HIP graphs of
    GRAPH_STEPS steps each (captured once; every replay follows an eager
    classification); then the split decode step replayed the same way for each
    n_split in `splits`."""
    import numpy as np
    import torch
    w, hk = gen_obj.w, gen_obj.hk
    d = w.head_dim
    cur = torch.cuda.current_stream()

    def classify():
        hk.hkv_classify(gen_obj.cfg, gen_obj.cache.state, gen_obj.K, gen_obj.V, w.N * d,
                        gen_obj.Q, w.q_rows * d, cur)

    def timed(body):
        out = []
        for k in range(steps + 1):                       # first one warms up
            classify()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(cur)
            body()
            b.record(cur)
            b.synchronize()
            if k:
                out.append(a.elapsed_time(b))
        hk.hkv_check(gen_obj.cfg, gen_obj.cache.state)
        return float(np.mean(out))

    def graphed(n_split):
        classify()
        torch.cuda.synchronize()
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(cur)
        t0 = time.perf_counter()
        for tb in range(w.P, w.N, GRAPH_STEPS):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                graph.capture_begin()
                decode_per_layer(gen_obj, side, n_split, tb, min(w.N, tb + GRAPH_STEPS))
                graph.capture_end()
            graphs.append(graph)
        torch.cuda.synchronize()
        capture_s = time.perf_counter() - t0

        def replay():
            for g in graphs:
                g.replay()
        ms = timed(replay)
        del graphs
        return ms, capture_s

    eager = timed(lambda: decode_per_layer(gen_obj, cur))
    replay, capture_s = graphed(0)
    layer_steps = w.steps * w.layers
    res = {"launches_per_step": w.layers, "streams_per_launch": w.batch * w.heads,
           "eager_ms_per_gen": round(eager, 3), "graph_ms_per_gen": round(replay, 3),
           "graph_tokens_per_s": round(w.batch * w.steps / (replay * 1e-3), 1),
           "graph_us_per_launch": round(replay * 1e3 / layer_steps, 3),
           "capture_s": round(capture_s, 2), "split": {}}
    for n in splits:
        ms, _ = graphed(n)
        res["split"][str(n)] = {"graph_ms_per_gen": round(ms, 3),
                                "graph_us_per_layer_step": round(ms * 1e3 / layer_steps, 3),
                                "graph_tokens_per_s": round(w.batch * w.steps / (ms * 1e-3), 1)}
    return res


def time_prefill(w, inputs, hk, full_cache_of, reps: int = 5) -> dict:
    """Classification alone (hkv_classify) against the prefill attention with
    the classification as its by-product (hkv_prefill), each with the initial
    layout, on the compressed and on the full-cache layout (where neither
    classifies, so the difference is the attention alone).  Prefill queries:
    seeded normal values on the device, the last W rows the workload's
    observation queries."""
    import numpy as np
    import torch
    K, V, Q = inputs
    S, P, d, N, W = w.S, w.P, w.head_dim, w.N, w.w_obs
    g = torch.Generator(device=K.device).manual_seed(7)
    qs = torch.randn((S, P, d), generator=g, device=K.device).to(K.dtype)
    qs[:, P - W:] = Q[:, :W]
    out = torch.empty((S, P, d), dtype=K.dtype, device=K.device)
    cur = torch.cuda.current_stream()

    def timed(fn):
        ms = []
        for k in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(cur)
            fn()
            b.record(cur)
            b.synchronize()
            if k:
                ms.append(a.elapsed_time(b))
        return float(np.mean(ms))

    res = {}
    for tag, wl in (("compressed", w), ("full_cache", full_cache_of(w))):
        cfg = hk.config_from_workload(wl)
        cache = hk.HkvCache(cfg)
        st = cache.state
        t_c = timed(lambda: hk.hkv_classify(cfg, st, K, V, N * d, Q, w.q_rows * d, cur))
        t_p = timed(lambda: hk.hkv_prefill(cfg, st, qs, P * d, K, V, N * d, out, P * d, cur))
        hk.hkv_check(cfg, st)
        res[tag] = {"classify_ms": round(t_c, 3), "prefill_ms": round(t_p, 3)}
        del cache
        torch.cuda.empty_cache()
    attn = res["full_cache"]["prefill_ms"] - res["full_cache"]["classify_ms"]
    byts = 4.0 * S * P * d * K.element_size()          # q, k, v read, output written
    res["attention_only_ms"] = round(attn, 3)
    res["fused_extra_ms"] = round(res["compressed"]["prefill_ms"] - res["compressed"]["classify_ms"], 3)
    res["attention_GBs"] = round(byts / (attn * 1e-3) / 1e9, 1) if attn > 0 else None
    res["attention_frac"] = round(byts / (attn * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if attn > 0 else None
    return res


def time_generations(gen_obj, steps, warmup, separate=False):
    """Mean ms per generation over `steps` timed generations, and the mean
    duration of one decode-step launch (HIP events bracketing each generation's
    decode loop on the launch stream, divided by the launches; the short gaps
    between consecutive launches are included)."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        gen_obj.run(stream, separate=separate)
        gen_obj.hk.hkv_check(gen_obj.cfg, gen_obj.cache.state, stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        gen_obj.run(stream, evs[k], separate=separate)
        # every generation's classification clears the device error word, so
        # each one is checked before the next starts
        gen_obj.hk.hkv_check(gen_obj.cfg, gen_obj.cache.state, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    loop_ms = np.array([a.elapsed_time(b) for a, b in evs])
    return wall / steps * 1e3, loop_ms / gen_obj.w.steps


def measure(w, inputs, hk, steps, warmup):
    """Timed generations of one workload: tokens/s over the whole generation
    and the dominant kernel's roofline figures (algorithmic bytes per launch /
    mean launch time from HIP events on the launch stream)."""
    import numpy as np
    gen_obj = Generation(w, inputs, hk)
    ms, launch_ms = time_generations(gen_obj, steps, warmup)
    labels = gen_obj.cache.label.cpu().numpy()
    budgets = gen_obj.cache.budget.cpu().numpy()
    alg = step_bytes(labels, budgets, w)
    kern_s = float(launch_ms.mean()) * 1e-3
    achieved = float(alg.mean()) / kern_s / 1e9
    return gen_obj, {"value": round(w.batch * w.steps / (ms * 1e-3), 1), "unit": "tokens/s",
                     "ms_per_step": round(ms, 4), "mean_launch_us": round(kern_s * 1e6, 3),
                     # the decode loop of each timed generation (HIP events): median, min
                     "launch_us_median": round(float(np.median(launch_ms)) * 1e3, 3),
                     "launch_us_min": round(float(launch_ms.min()) * 1e3, 3),
                     "alg_bytes_per_launch": round(float(alg.mean()), 1),
                     "achieved_GBs": round(achieved, 1),
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "labels": {"local": int((labels == 0).sum()),
                                "global": int((labels == 1).sum())}}


def levels(gen_obj, steps):
    """The decode step measured at its two levels: the fused launch (measured
    above) and the same step as three separate calls, whose middle one is the
    attention kernel alone.  HIP events bracket each generation's decode loop;
    the per-kernel split of the separate calls comes from a kernel trace
    (rocprofv3), since events around single launches would add their own gaps.
    This reports the loop time per decode step and the attention launch's
    algorithmic bytes, from which the trace's attention duration gives its
    fraction of peak."""
    w = gen_obj.w
    ms, launch_ms = time_generations(gen_obj, steps, 1, separate=True)
    labels = gen_obj.cache.label.cpu().numpy()
    budgets = gen_obj.cache.budget.cpu().numpy()
    a = attn_bytes(labels, budgets, w)
    return {"separate_calls": {"ms_per_step": round(ms, 4),
                               "us_per_decode_step": round(float(launch_ms.mean()) * 1e3, 3),
                               "launches_per_decode_step": 3,
                               "attn_alg_bytes_per_launch": round(float(a.mean()), 1),
                               "attn_kernel": "k_step<AP=false, AT=true, EV=false> "
                                              "(hkv_decode_attn)"}}


def fidelity(comp, full):
    """Relative L2 error of every compressed attention output against the
    full-cache output of the same stream and step (one untimed generation each)."""
    import torch
    w = comp.w
    stream = torch.cuda.current_stream()
    a = torch.empty((w.steps, w.S, w.head_dim), dtype=comp.K.dtype, device=comp.K.device)
    b = torch.empty_like(a)
    comp.run(stream, capture=a)
    full.run(stream, capture=b)
    torch.cuda.synchronize()
    a32, b32 = a.float(), b.float()
    rel = (a32 - b32).norm(dim=-1) / b32.norm(dim=-1).clamp_min(1e-30)
    q = torch.quantile(rel.flatten()[:: max(1, rel.numel() // 1_000_000)],
                       torch.tensor([0.5, 0.99], device=rel.device))
    return {"rel_l2_mean": round(float(rel.mean()), 6), "rel_l2_median": round(float(q[0]), 6),
            "rel_l2_p99": round(float(q[1]), 6), "rel_l2_max": round(float(rel.max()), 6),
            "what": "compressed vs full-cache attention output, every stream and step"}


VARIANTS = {"headkv": (False, False), "unstratified": (True, False),
            "uniform_budget": (False, True), "uniform_unstratified": (True, True)}


def copy_bandwidth(gib: int = 4, reps: int = 5) -> float:
    """Achieved bandwidth of a plain device-to-device copy of `gib` GiB (bytes
    read + written per second, best of `reps`): the practical HBM ceiling the
    kernel's rate is also compared with."""
    import torch
    n = gib << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        e1.synchronize()
        best = max(best, 2.0 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del a, b
    torch.cuda.empty_cache()
    return best


def copy_calibration():
    """A plain device copy of known size, for scaling the HBM counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n, "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llamagen_xl_rho1_6")
    ap.add_argument("--second", default="janus_pro_7b_rho1_6",
                    help="a second workload measured the same way in the same run "
                         "(compressed layout only; '' to skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full-cache", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--variant", default="headkv", choices=sorted(VARIANTS),
                    help="ablation: eviction without the near/far split and/or one budget "
                         "for every head")
    ap.add_argument("--fidelity", action="store_true",
                    help="also report the attention-output error against the full cache")
    ap.add_argument("--per-layer", action="store_true",
                    help="also time the per-layer decode loop, eager and as a HIP graph")
    ap.add_argument("--jsonl", default="",
                    help="also append the result, with a timestamp and the kernel sources' hash, "
                         "to this JSONL file (a per-run log)")
    ap.add_argument("--per-layer-splits", default="2,4,8",
                    help="n_split values of the split decode step timed with --per-layer")
    ap.add_argument("--prefill", action="store_true",
                    help="also time hkv_prefill (prefill attention with the classification as "
                         "its by-product) against hkv_classify")
    ap.add_argument("--levels", action="store_true",
                    help="also time the decode step as three separate calls (append, "
                         "attention, eviction): the attention kernel alone is the middle one")
    ap.add_argument("--e2e", action="store_true",
                    help="also time a random-weight transformer of the backbone's shape around "
                         "the decode path, compressed and full cache (bench_e2e.py)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode path is per-stream independent "
              "and this build runs on a single MI355X; use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import kv_cache_compression_hkv_amd as hk
    from hkv_inputs.configs import WORKLOADS, full_cache_of, variant_of
    from hkv_inputs.gpu import device_inputs

    if args.copy_calibration:
        copy_calibration()
        return

    w = WORKLOADS[args.workload]
    if args.variant != "headkv":
        w = variant_of(w, *VARIANTS[args.variant])
    torch.cuda.set_device(0)
    inputs = device_inputs(w, args.seed)

    comp, m = measure(w, inputs, hk, args.steps, args.warmup)
    ms = m["ms_per_step"]
    kern_mean_s = m["mean_launch_us"] * 1e-6
    achieved = m["achieved_GBs"]
    tokens = w.batch * w.steps
    value = m["value"]

    copy_gbs = copy_bandwidth()
    traffic = None
    if os.path.exists(COUNTERS_FILE):
        with open(COUNTERS_FILE) as f:
            cnt = json.load(f)
        if cnt.get("kernel_hash") == kernel_hash() and cnt.get("workload") == w.name:
            traffic = cnt.get("hbm_bytes_per_launch")

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "batch": w.batch, "heads": w.heads,
                   "head_dim": w.head_dim, "final_len": w.N, "prefill_len": w.P,
                   "rho": f"{w.rho[0]}/{w.rho[1]}", "decode_steps": w.steps,
                   "launch": "layer-folded, 1 fused launch per decode step",
                   "variant": args.variant,
                   "global_batch": w.batch, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": m["frac"],
                     "traffic": traffic,
                     "kernel": "k_step (fused append + attention + STE)",
                     "mean_launch_us": m["mean_launch_us"],
                     "launch_us_median": m["launch_us_median"],
                     "launch_us_min": m["launch_us_min"],
                     "alg_bytes_per_launch": m["alg_bytes_per_launch"],
                     "copy_GBs": round(copy_gbs, 1),
                     "frac_of_copy": round(achieved / copy_gbs, 4)},
        "labels": m["labels"],
    }
    if args.levels:
        res["levels"] = levels(comp, max(2, args.steps // 2))
    if args.per_layer:
        splits = tuple(int(x) for x in args.per_layer_splits.split(",") if x)
        res["per_layer"] = time_per_layer(comp, max(2, args.steps // 2), splits)
    if args.prefill and w.dtype == "bf16":
        res["prefill"] = time_prefill(w, inputs, hk, full_cache_of)
    if not args.no_full_cache:
        wf = full_cache_of(w)
        full = Generation(wf, inputs, hk)
        if args.fidelity:
            res["fidelity"] = fidelity(comp, full)
        del comp
        torch.cuda.empty_cache()
        ms_f, launch_f = time_generations(full, max(2, args.steps // 2), 1)
        lab_f = full.cache.label.cpu().numpy()
        alg_f = step_bytes(lab_f, full.cache.budget.cpu().numpy(), wf)
        kf = float(launch_f.mean()) * 1e-3
        res["full_cache"] = {"value": round(tokens / (ms_f * 1e-3), 1), "ms_per_step": round(ms_f, 4),
                             "mean_launch_us": round(kf * 1e6, 3),
                             "achieved_GBs": round(float(alg_f.mean()) / kf / 1e9, 1),
                             "speedup_step": round(ms_f / ms, 3),
                             "speedup_kernel": round(kf / kern_mean_s, 3)}
        del full
    if args.second and args.second != w.name:
        # the second rho = 1/6 workload, same protocol (compressed layout only)
        comp = None
        torch.cuda.empty_cache()
        w2 = WORKLOADS[args.second]
        if args.variant != "headkv":
            w2 = variant_of(w2, *VARIANTS[args.variant])
        inputs2 = device_inputs(w2, args.seed)
        g2, m2 = measure(w2, inputs2, hk, args.steps, args.warmup)
        m2["workload"] = w2.name
        m2["rho"] = f"{w2.rho[0]}/{w2.rho[1]}"
        res["second_workload"] = m2
        del g2, inputs2
        torch.cuda.empty_cache()
    if args.e2e:
        import bench_e2e
        comp = None
        torch.cuda.empty_cache()
        res["e2e"] = bench_e2e.run(w, args.seed, max(1, args.steps // 4), hk, device_inputs,
                                   full_cache_of)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.seed)
    line = json.dumps(res)
    if args.jsonl:
        # the run's record, appended with when and with which kernel sources it ran
        rec = dict(res, time_utc=time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime()),
                   kernel_hash=kernel_hash(), argv=sys.argv[1:])
        with open(args.jsonl, "a") as f:
            f.write(json.dumps(rec) + "\n")
    print(line, flush=True)


if __name__ == "__main__":
    main()
