"""End-to-end decode throughput of a random-weight autoregressive transformer
built around the HeadKV decode path (one MI355X).

The pages report whole-model speedups of image-generation backbones (section
"Results": 3.00x on LlamaGen-XL, 3.68x on Janus-Pro-7B at rho = 1/6, 1.35x on
Lumina-mGPT-768).  This driver is a weights-free analogue: the backbone's layer
count, heads and head size, a pre-norm block with a SwiGLU MLP, random weights,
and per layer per decode step

    x -> RMSNorm -> q, k, v GEMMs -> hkv_decode_step over the layer's batch x heads
      streams (append, attention, eviction) -> output GEMM -> residual
      -> RMSNorm -> gate/up GEMM -> SiLU * up -> down GEMM -> residual,

then RMSNorm -> LM-head GEMM -> greedy token -> embedding of the next step.  The
pages do not give the backbones' MLP widths or vocabularies; the public
intermediate sizes and image vocabularies below are an assumption, and rotary
position encoding is left out (it does not change the bytes moved).  Prefill is
synthetic: the seeded K, V and observation queries of the workload, as in the
decode benchmark, feed hkv_classify; the decode loop then runs on the model's
own activations.

The decode loop is captured once as HIP graphs of CHUNK decode steps each
(tens of thousands of nodes per graph; a whole generation's several hundred
thousand in one graph is more than the runtime's instantiation handles) and
replayed in order after an eager classification, so Python does not pace it.  The
same loop without the hkv_decode_step calls gives the time of everything else;
the difference is the attention's share.  Run for the compressed cache and for
the full-cache layout of the same workload.
"""
from __future__ import annotations

import math
import sys
import time

# decode steps per captured graph: about 9e3 graph nodes at LlamaGen-XL's 36
# layers.  A whole generation (about 3e5 nodes) in one graph ended the process
# during instantiation, so graphs stay bounded by this.
CHUNK = 16

# generation-side width of each backbone: (MLP intermediate size, vocabulary)
ARCH = {
    "llamagen_xl": (3584, 16384),
    "janus_pro_1b": (5632, 16384),
    "janus_pro_7b": (11008, 16384),
    "lumina_mgpt_768": (11008, 65536),
    "tiny": (512, 1024),
}


def arch_of(name: str):
    for k, v in ARCH.items():
        if name.startswith(k):
            return v
    raise KeyError(name)


class Model:
    """Random weights (seeded) of the backbone's decoder, stored [in, out]."""

    def __init__(self, w, seed: int, device):
        import torch
        self.w = w
        H, d, L = w.heads, w.head_dim, w.layers
        self.hid = hid = H * d
        self.mlp, self.vocab = arch_of(w.name)
        self.dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        g = torch.Generator(device=device).manual_seed(seed)

        def mat(i, o):
            m = torch.randn(i, o, generator=g, device=device, dtype=torch.float32)
            return (m / math.sqrt(i)).to(self.dt)

        self.wq = [mat(hid, hid) for _ in range(L)]
        self.wk = [mat(hid, hid) for _ in range(L)]
        self.wv = [mat(hid, hid) for _ in range(L)]
        self.wo = [mat(hid, hid) for _ in range(L)]
        self.wgu = [mat(hid, 2 * self.mlp) for _ in range(L)]
        self.wd = [mat(self.mlp, hid) for _ in range(L)]
        self.g1 = [torch.ones(hid, device=device, dtype=self.dt) for _ in range(L)]
        self.g2 = [torch.ones(hid, device=device, dtype=self.dt) for _ in range(L)]
        self.gf = torch.ones(hid, device=device, dtype=self.dt)
        self.emb = (torch.randn(self.vocab, hid, generator=g, device=device) * 0.02).to(self.dt)
        self.wlm = mat(hid, self.vocab)

    def param_bytes(self) -> int:
        ts = (self.wq + self.wk + self.wv + self.wo + self.wgu + self.wd +
              [self.emb, self.wlm])
        return sum(t.numel() * t.element_size() for t in ts)


def rmsnorm(x, g, eps=1e-6):
    import torch
    return torch.nn.functional.rms_norm(x, (x.shape[-1],), g, eps)


class Driver:
    """One generation of the model over the HeadKV cache of workload `w`."""

    def __init__(self, w, model: Model, inputs, hk):
        import torch
        self.w, self.m, self.hk = w, model, hk
        self.K, self.V, self.Q = inputs
        self.cfg = hk.config_from_workload(w)
        self.cache = hk.HkvCache(self.cfg)
        dev = self.K.device
        B, H, d, W = w.batch, w.heads, w.head_dim, w.w_obs
        self.per = B * H
        self.eb = self.K.element_size()
        hid = model.hid
        # fixed buffers, so the captured graph's pointers stay valid
        self.tok = torch.zeros(B, dtype=torch.long, device=dev)
        self.x = torch.zeros(B, hid, dtype=model.dt, device=dev)
        self.h = torch.empty(B, hid, dtype=model.dt, device=dev)
        self.q = torch.empty(B, hid, dtype=model.dt, device=dev)
        self.k = torch.empty(B, hid, dtype=model.dt, device=dev)
        self.v = torch.empty(B, hid, dtype=model.dt, device=dev)
        self.att = torch.empty(B, hid, dtype=model.dt, device=dev)
        self.gu = torch.empty(B, 2 * model.mlp, dtype=model.dt, device=dev)
        self.logits = torch.empty(B, model.vocab, dtype=model.dt, device=dev)
        # per layer, the W newest queries of every stream in a doubled ring:
        # position p sits in slots p mod W and p mod W + W, so the window
        # t-W+1 .. t is the contiguous run starting at slot (t + 1) mod W
        self.qring = [torch.zeros(self.per, 2 * W, d, dtype=model.dt, device=dev)
                      for _ in range(w.layers)]
        self.rec = None     # optional recording of one (layer, sequence) group

    def record(self, layer: int, seq: int, on_classified=None):
        """One eager generation that keeps, for the streams of (layer, seq), the
        rows handed to hkv_decode_step at every step (k, v, the newest query)
        with its output and evicted positions, for a replay on another
        implementation.  `on_classified()` runs between the classification and
        the first step.  Returns the recording (device tensors)."""
        import torch
        w, dev = self.w, self.K.device
        H, d, T, M = w.heads, w.head_dim, w.steps, w.evict_m
        lo = seq * H                               # the group's rows inside the layer
        rec = {"layer": layer, "rows": slice(lo, lo + H),
               "k": torch.empty(T, H, d, dtype=self.m.dt, device=dev),
               "v": torch.empty(T, H, d, dtype=self.m.dt, device=dev),
               "q": torch.empty(T, H, d, dtype=self.m.dt, device=dev),
               "out": torch.empty(T, H, d, dtype=self.m.dt, device=dev),
               "log_all": torch.full((w.S, M), -1, dtype=torch.int32, device=dev),
               "log": torch.empty(T, H, M, dtype=torch.int32, device=dev)}
        self.rec = rec
        try:
            self._reset()
            if on_classified is not None:
                torch.cuda.synchronize()
                on_classified()
            self._loop(True)
        finally:
            self.rec = None
        torch.cuda.synchronize()
        return rec

    def _reset(self):
        """Eager: classification from the synthetic prefill, first token, query
        rings seeded with the last prefill queries."""
        import torch
        w, hk, d, W = self.w, self.hk, self.w.head_dim, self.w.w_obs
        hk.hkv_classify(self.cfg, self.cache.state, self.K, self.V, w.N * d, self.Q,
                        w.q_rows * d)
        self.tok.zero_()
        for l in range(w.layers):
            # row r of Q holds position P-W+r; the first step's window needs
            # positions P-W+1 .. P-1 besides its own query
            rows = self.Q[l * self.per:(l + 1) * self.per, 1:W]
            for i in range(W - 1):
                p = w.P - W + 1 + i
                self.qring[l][:, p % W] = rows[:, i]
                self.qring[l][:, p % W + W] = rows[:, i]

    def _loop(self, attention: bool, t_begin=None, t_end=None):
        """Decode steps t_begin .. t_end-1, by default all of P .. N-1
        (graph-capturable: device work only)."""
        import torch
        w, m, hk, st = self.w, self.m, self.hk, self.cache.state
        d, W, eb, per = w.head_dim, w.w_obs, self.eb, self.per
        t_begin = w.P if t_begin is None else t_begin
        t_end = w.N if t_end is None else t_end
        for t in range(t_begin, t_end):
            torch.index_select(m.emb, 0, self.tok, out=self.x)
            for l in range(w.layers):
                self.h.copy_(rmsnorm(self.x, m.g1[l]))
                torch.matmul(self.h, m.wq[l], out=self.q)
                torch.matmul(self.h, m.wk[l], out=self.k)
                torch.matmul(self.h, m.wv[l], out=self.v)
                qv = self.q.view(per, d)
                self.qring[l][:, t % W] = qv
                self.qring[l][:, t % W + W] = qv
                if attention:
                    s0 = l * per                       # this layer's first stream
                    kp = self.k.data_ptr() - s0 * d * eb
                    vp = self.v.data_ptr() - s0 * d * eb
                    qw = self.qring[l].data_ptr() + ((t + 1) % W) * d * eb - s0 * 2 * W * d * eb
                    op = self.att.data_ptr() - s0 * d * eb
                    rec = self.rec if (self.rec is not None and self.rec["layer"] == l) else None
                    hk.hkv_decode_step(self.cfg, st, t, kp, vp, d, qw, 2 * W * d, op, d,
                                       None if rec is None else rec["log_all"], s0, per,
                                       torch.cuda.current_stream())
                    if rec is not None:
                        r, i = rec["rows"], t - w.P
                        rec["k"][i] = self.k.view(per, d)[r]
                        rec["v"][i] = self.v.view(per, d)[r]
                        rec["q"][i] = qv[r]
                        rec["out"][i] = self.att.view(per, d)[r]
                        rec["log"][i] = rec["log_all"][s0 + r.start:s0 + r.stop]
                else:
                    self.att.copy_(self.v)
                self.x.add_(self.att @ m.wo[l])
                torch.matmul(rmsnorm(self.x, m.g2[l]), m.wgu[l], out=self.gu)
                g, u = self.gu.split(m.mlp, dim=1)
                self.x.add_((torch.nn.functional.silu(g) * u) @ m.wd[l])
            torch.matmul(rmsnorm(self.x, m.gf), m.wlm, out=self.logits)
            torch.argmax(self.logits, dim=-1, out=self.tok)

    def time(self, reps: int, attention: bool = True) -> dict:
        """Mean ms per generation's decode loop, replayed from captured graphs."""
        import numpy as np
        import torch
        w = self.w
        tag = f"e2e {w.name} attention={attention}"
        cur = torch.cuda.current_stream()
        print(f"[{tag}] eager warm-up", file=sys.stderr, flush=True)
        self._reset()
        self._loop(attention)                          # eager warm-up (allocator, kernels)
        torch.cuda.synchronize()
        self._reset()
        torch.cuda.synchronize()
        print(f"[{tag}] capture ({w.steps} steps, {CHUNK} per graph)", file=sys.stderr, flush=True)
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(cur)
        t0 = time.perf_counter()
        for tb in range(w.P, w.N, CHUNK):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                g.capture_begin()
                self._loop(attention, tb, min(w.N, tb + CHUNK))
                g.capture_end()
            graphs.append(g)
        torch.cuda.synchronize()
        capture_s = time.perf_counter() - t0
        print(f"[{tag}] replay", file=sys.stderr, flush=True)
        ms = []
        for k in range(reps + 1):                      # first replay warms up
            self._reset()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(cur)
            for g in graphs:
                g.replay()
            b.record(cur)
            b.synchronize()
            if k:
                ms.append(a.elapsed_time(b))
        if attention:
            self.hk.hkv_check(self.cfg, self.cache.state)
        del graphs
        return {"ms_per_gen": float(np.mean(ms)), "capture_s": capture_s}


def run(w, seed: int, reps: int, hk, device_inputs, full_cache_of) -> dict:
    """Compressed and full-cache end-to-end decode throughput for workload w."""
    import torch
    model = Model(w, seed, torch.device("cuda"))
    res = {"model": {"layers": w.layers, "heads": w.heads, "head_dim": w.head_dim,
                     "hidden": model.hid, "mlp": model.mlp, "vocab": model.vocab,
                     "weights_GB": round(model.param_bytes() / 1e9, 2), "batch": w.batch,
                     "decode_steps": w.steps}}
    base = None
    for tag, wl in (("compressed", w), ("full_cache", full_cache_of(w))):
        drv = Driver(wl, model, device_inputs(wl, seed), hk)
        t_all = drv.time(reps, attention=True)
        if base is None:
            base = drv.time(reps, attention=False)["ms_per_gen"]   # the same without attention
        ms = t_all["ms_per_gen"]
        res[tag] = {"tokens_per_s": round(wl.batch * wl.steps / (ms * 1e-3), 1),
                    "ms_per_gen": round(ms, 3),
                    "attention_ms": round(ms - base, 3),
                    "capture_s": round(t_all["capture_s"], 2)}
        del drv
        torch.cuda.empty_cache()
    res["rest_ms"] = round(base, 3)
    res["speedup"] = round(res["full_cache"]["ms_per_gen"] / res["compressed"]["ms_per_gen"], 3)
    res["attention_speedup"] = round(res["full_cache"]["attention_ms"] /
                                     max(1e-9, res["compressed"]["attention_ms"]), 3)
    return res
