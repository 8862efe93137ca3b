#!/usr/bin/env python3
"""MoE layer forward benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--T T]

A step is one pass of the whole layer (router, gating, histogram, prefix sum,
permutation, grouped SwiGLU GEMMs, shared expert if any, combine) over one
batch of T seeded synthetic tokens, through the fused C entry point
moe_layer.  Inputs are resident in HBM before the timed region.  Steps
rotate over byte-identical copies of the layer's weights at distinct
addresses, as many as make the bytes the rotation touches (the router and
the experts the batch actually routes to, per copy) at least 1 GB, four
times the 256 MB Infinity Cache, so no step finds its weights in that cache.

Printed: one JSON line with tokens/s (value), the roofline of the dominant
kernel (timed live with HIP events that moe_layer records on its stream at
stage boundaries), the whole-layer roofline fraction, a per-stage time split,
a graph-replayed sweep over the workload's other token counts, and the CPU
oracle timed on a bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s and % roofline (HBM GB/s at decode, MFMA at prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X fp32 (vector/matrix) for the fp32 layer
WORKLOAD_NAMES = {
    "toy_f32": "toy_moe_layer_f32",
    "mixtral_8x7b": "mixtral_8x7b_moe_layer",
    "qwen3_ep_all128": "qwen3_235b_a22b_moe_layer_ep_all128",
    "qwen3_tp8_rank0": "qwen3_235b_a22b_moe_layer_tp8_rank0",
    "deepseek_v3": "deepseek_v3_moe_layer_shared1",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_ep_all128", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--T", type=int, default=None, help="tokens per step (default: largest of the workload)")
    ap.add_argument("--copies", type=int, default=None, help="weight copies to rotate over")
    ap.add_argument("--path", default="auto", choices=["auto", "staged", "decode"],
                    help="layer entry point: moe_layer (auto), moe_layer_staged, moe_layer_decode")
    ap.add_argument("--no-sweep", action="store_true", help="skip the token-count sweep")
    ap.add_argument("--sweep-workloads",
                    default="qwen3_ep_all128,qwen3_tp8_rank0,mixtral_8x7b,deepseek_v3",
                    help="workloads whose token counts are swept (comma list)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dispatch", action="store_true",
                    help="skip the expert-parallel dispatch packing measurement")
    ap.add_argument("--no-reshard", action="store_true",
                    help="skip the EP <-> TP weight reshard measurement")
    ap.add_argument("--no-capacity", action="store_true",
                    help="skip the capacity-factor (token dropping) measurement")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens in the CPU oracle sample (default: the whole batch)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the CPU oracle repeats whole passes over its sample until this much "
                         "time has been spent")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB read + 1 GiB write elementwise kernel 3 times "
                         "(calibrates the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (bytes / FLOPs the method itself must move or compute)
# ---------------------------------------------------------------------------

def layer_work(cfg, T, counts, I_loc, elt):
    rows = int(sum(counts))
    touched = int(sum(1 for c in counts if c > 0))
    H, E = cfg.H, cfg.E
    w_bytes = elt * (E * H + touched * 3 * I_loc * H + 3 * cfg.I_shared * H)
    b_alg = w_bytes + 2 * elt * T * H
    f_alg = 2 * T * E * H + 6 * rows * I_loc * H + 6 * T * cfg.I_shared * H
    g1_flops = 4 * rows * I_loc * H
    g1_bytes = elt * (touched * 2 * I_loc * H + T * H + rows * I_loc)
    return dict(rows=rows, touched=touched, b_alg=b_alg, f_alg=f_alg, g1_flops=g1_flops,
                g1_bytes=g1_bytes)


ROTATION_BYTES = 1.0e9     # bytes the weight rotation must touch (>= 4x the 256 MB MALL)
MAX_COPIES = 64


def copies_needed(cfg, work, T, elt):
    """Weight copies for a batch: enough that copies x (bytes one step
    touches: router + routed experts + shared expert) >= ROTATION_BYTES."""
    touched = work["b_alg"] - 2 * elt * T * cfg.H
    return max(2, min(MAX_COPIES, math.ceil(ROTATION_BYTES / max(touched, 1))))


def routing_shape(counts, T, k, E):
    """The expert-GEMM shape distribution of a batch: rows per expert (m),
    their percentiles and maximum, the imbalance max / mean over all experts,
    and a histogram of m over power-of-two bins."""
    import numpy as np
    c = np.asarray(counts, dtype=np.int64)
    rows = int(c.sum())
    mean = rows / max(len(c), 1)
    hist = {}
    for m in c.tolist():
        key = "0" if m == 0 else f"{1 << (m.bit_length() - 1)}-{(1 << m.bit_length()) - 1}"
        hist[key] = hist.get(key, 0) + 1
    order = sorted(hist, key=lambda s: int(s.split("-")[0]))
    return dict(rows=rows, touched_experts=int((c > 0).sum()),
                imbalance_ratio=round(float(c.max() / mean), 3) if rows else 0.0,
                load_p50=float(np.percentile(c, 50)), load_p95=float(np.percentile(c, 95)),
                load_p99=float(np.percentile(c, 99)), load_max=int(c.max()),
                m_hist={key: hist[key] for key in order})


def roofs(cfg):
    if cfg.dtype == "f32":
        return HBM_PEAK_GBS, MFMA_F32_PEAK_TFLOPS
    return HBM_PEAK_GBS, MFMA_BF16_PEAK_TFLOPS


# ---------------------------------------------------------------------------
# GPU setup
# ---------------------------------------------------------------------------

LAYER_FN = {"auto": "moe_layer", "staged": "moe_layer_staged", "decode": "moe_layer_decode"}


class Bench:
    """One workload's layer on the GPU: weights (with copies for the
    rotation), workspace, input batch.  `copies` fixes the rotation length;
    None sizes it per batch from the touched bytes (copies_needed)."""

    def __init__(self, name, T_max, copies, path="auto"):
        import torch
        import mixture_experts_layer_amd as M
        import workloads as W
        self.torch, self.M, self.W = torch, M, W
        self.layer_fn = getattr(M, LAYER_FN[path])
        self.cfg = cfg = W.CONFIGS[name]
        L = W.make_layer(cfg, device="cuda", seed=0, T_max=T_max)
        w13, w2 = W.share_weights(L.w13, L.w2, cfg.tp_P, cfg.tp_rank)
        L.w13 = L.w2 = None
        torch.cuda.empty_cache()
        self.L = L
        self.elt = 4 if cfg.dtype == "f32" else 2
        self.I_loc = w13.shape[1] // 2
        self.fixed_copies = copies
        self.layers = []
        self._add_copy(w13, w2, L.w_r, L.w13_shared, L.w2_shared)
        self.copies = 1
        self.T_max = T_max
        self.ws = M.layer_workspace(self.layers[0][0], T_max)
        self.ws_bytes = self.ws.numel()
        self.y_full = torch.empty((T_max, cfg.H), dtype=L.x.dtype, device="cuda")
        self.set_T(T_max)
        torch.cuda.synchronize()

    def _add_copy(self, w13, w2, w_r, w13_s, w2_s):
        cfg, M, L = self.cfg, self.M, self.L
        d = self.M.layer_desc(cfg.H, cfg.E, cfg.k, self.I_loc, cfg.mode, M.dtype_code(L.x), w_r,
                              w13, w2, I_shared=cfg.I_shared, w13_shared=w13_s, w2_shared=w2_s,
                              logit_bias=L.logit_bias, sel_bias=L.sel_bias)
        self.layers.append((d, w13, w2, w_r, w13_s, w2_s))

    def set_copies(self, n):
        """Rotate over n copies of every weight the layer reads (router,
        experts, shared expert), cloning more if needed."""
        _, w13, w2, w_r, w13_s, w2_s = self.layers[0]
        clone = lambda t: None if t is None else t.clone()
        while len(self.layers) < n:
            self._add_copy(clone(w13), clone(w2), clone(w_r), clone(w13_s), clone(w2_s))
        self.copies = n

    def size_rotation(self, work):
        """Set the rotation for the current batch from its touched bytes."""
        n = self.fixed_copies or copies_needed(self.cfg, work, self.T, self.elt)
        self.set_copies(n)
        return n

    def set_T(self, T):
        self.T = T
        self.x = self.L.x[:T]
        self.y = self.y_full[:T]

    def counts(self):
        torch, M = self.torch, self.M
        E_loc = self.cfg.E_loc
        counts = torch.empty((E_loc,), dtype=torch.int32, device="cuda")
        dbg = M.debug_out(counts=counts)
        self.layer_fn(self.layers[0][0], self.T, self.x, self.y, self.ws, self.ws_bytes, dbg)
        torch.cuda.synchronize()
        return counts.cpu().tolist()

    def path_of(self, T):
        """The path the timed entry point takes at T ("decode" or "staged")."""
        if self.layer_fn is self.M.moe_layer:
            return self.M.moe_layer_path(self.layers[0][0], T)
        return "decode" if self.layer_fn is self.M.moe_layer_decode else "staged"

    def step(self, i, dbg=None):
        d = self.layers[i % self.copies][0]
        self.layer_fn(d, self.T, self.x, self.y, self.ws, self.ws_bytes, dbg)

    def timed_eager(self, steps, warmup):
        """Exactly `steps` eager layer calls; every call records the six stage
        events on the library's stream."""
        torch, M = self.torch, self.M
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
        for row in evs:
            for e in row:
                e.record()          # materialise the underlying hipEvent_t
        dbgs = [M.debug_out(stage_events=[e.cuda_event for e in row]) for row in evs]
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i, dbgs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = (t1 - t0) * 1e3 / steps
        names = ["route_permute", "gemm_gate_up", "gemm_down", "shared_expert", "combine"]
        split = {n: sum(r[j].elapsed_time(r[j + 1]) for r in evs) / steps for j, n in enumerate(names)}
        return ms, split

    def timed_graph(self, steps, warmup):
        """Layer time from replays of a HIP graph holding one layer call per
        weight copy (launch overhead amortised, as graph-replayed decode)."""
        torch = self.torch
        for i in range(max(warmup, 2)):
            self.step(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(self.copies):
                self.step(c)
        reps = max(1, math.ceil(steps / self.copies))
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        self.graph_event_ms = e0.elapsed_time(e1) / (reps * self.copies)
        return (t1 - t0) * 1e3 / (reps * self.copies)


def roofline_entry(cfg, work, t_g1_ms):
    hbm, mfma = roofs(cfg)
    ai = work["g1_flops"] / max(work["g1_bytes"], 1)
    ridge = mfma * 1e12 / (hbm * 1e9)
    if ai >= ridge:
        ach = work["g1_flops"] / (t_g1_ms * 1e-3) / 1e12
        return dict(bound="mfma", achieved=round(ach, 2), peak=mfma, unit="TFLOP/s",
                    frac=round(ach / mfma, 4), traffic=None)
    ach = work["g1_bytes"] / (t_g1_ms * 1e-3) / 1e9
    return dict(bound="hbm", achieved=round(ach, 1), peak=hbm, unit="GB/s",
                frac=round(ach / hbm, 4), traffic=None)


def decode_roofline_entry(cfg, work, t_ms):
    """Roofline of the single-launch decode kernel: the whole layer's
    algorithmic bytes (or FLOPs, past the ridge) over the kernel's time."""
    hbm, mfma = roofs(cfg)
    if work["b_alg"] / (hbm * 1e9) >= work["f_alg"] / (mfma * 1e12):
        ach = work["b_alg"] / (t_ms * 1e-3) / 1e9
        return dict(bound="hbm", achieved=round(ach, 1), peak=hbm, unit="GB/s",
                    frac=round(ach / hbm, 4), traffic=None)
    ach = work["f_alg"] / (t_ms * 1e-3) / 1e12
    return dict(bound="mfma", achieved=round(ach, 2), peak=mfma, unit="TFLOP/s",
                frac=round(ach / mfma, 4), traffic=None)


def layer_roof_frac(cfg, work, ms):
    hbm, mfma = roofs(cfg)
    t_roof = max(work["b_alg"] / (hbm * 1e9), work["f_alg"] / (mfma * 1e12))
    bound = "hbm" if work["b_alg"] / (hbm * 1e9) >= work["f_alg"] / (mfma * 1e12) else "mfma"
    return bound, t_roof * 1e3, t_roof / (ms * 1e-3)


# ---------------------------------------------------------------------------
# Expert-parallel dispatch packing (the source rank's side of the exchange)
# ---------------------------------------------------------------------------

def dispatch_bench(steps, warmup, P=8, Ts=(64, 4096)):
    """moe_pack_by_rank (copies by destination rank + their x rows) and
    moe_unpack_sum (the sum of the returned rows) on the DeepSeek-V3-shaped
    layer's routing, as one of P expert-parallel ranks would run them, timed
    by HIP-graph replay.  Algorithmic bytes: pack reads x once per token and
    the routing, writes every copy's row and routing; unpack reads every
    returned row once and writes y."""
    import torch
    import mixture_experts_layer_amd as M
    import workloads as W
    cfg = W.CONFIGS["deepseek_v3"]
    T_max = max(Ts)
    L = W.make_layer(cfg, device="cuda", seed=0, T_max=T_max, experts=False)
    H, E, k = cfg.H, cfg.E, cfg.k
    dt = M.dtype_code(L.x)
    logits = torch.empty((T_max, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T_max, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T_max, k), dtype=torch.float32, device="cuda")
    M.moe_route(L.x, L.w_r, dt, T_max, H, E, k, cfg.mode, L.logit_bias, L.sel_bias, logits, ids, w)
    rows_max = T_max * min(k, P)
    counts = torch.empty((P,), dtype=torch.int32, device="cuda")
    offsets = torch.empty((P + 1,), dtype=torch.int32, device="cuda")
    send_token = torch.empty((rows_max,), dtype=torch.int32, device="cuda")
    send_row = torch.empty((T_max, k), dtype=torch.int32, device="cuda")
    send_ids = torch.empty((rows_max, k), dtype=torch.int32, device="cuda")
    send_w = torch.empty((rows_max, k), dtype=torch.float32, device="cuda")
    x_send = torch.empty((rows_max, H), dtype=L.x.dtype, device="cuda")
    y = torch.empty((T_max, H), dtype=L.x.dtype, device="cuda")
    nb = M.moe_pack_workspace_size(T_max, k, P)
    ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
    out = []
    for T in Ts:
        def pack():
            M.moe_pack_by_rank(ids, w, T, k, E, P, L.x, H, dt, counts, offsets, send_token,
                               send_row, send_ids, send_w, x_send, ws, nb)

        def unpack():
            M.moe_unpack_sum(x_send, dt, send_row, T, k, H, y, dt)

        pack()
        torch.cuda.synchronize()
        rows = int(offsets[P].item())
        res = dict(workload="deepseek_v3_moe_layer_shared1 routing, one of %d expert-parallel ranks"
                   % P, T=T, P=P, copies=rows,
                   copies_to_other_ranks_per_token=None)
        for name, fn, nbytes in (
                ("pack_by_rank", pack, 2 * T * H + T * k * 8 + rows * (2 * H + 8 * k + 4) + T * k * 4),
                ("unpack_sum", unpack, rows * 2 * H + T * 2 * H + T * k * 4)):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(10):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, steps // 10)
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / (reps * 10)
            gbs = nbytes / (ms * 1e-3) / 1e9
            res[name] = dict(ms=round(ms, 4), algorithmic_bytes=int(nbytes),
                             achieved_GBs=round(gbs, 1), peak_GBs=HBM_PEAK_GBS,
                             frac=round(gbs / HBM_PEAK_GBS, 4))
        c = counts.cpu().tolist()
        # rank 0 stands for the source's own rank
        res["copies_to_other_ranks_per_token"] = round((rows - c[0]) / T, 3)
        out.append(res)
        print(f"# dispatch T={T}: pack {res['pack_by_rank']['ms']} ms "
              f"({res['pack_by_rank']['frac']}), unpack {res['unpack_sum']['ms']} ms "
              f"({res['unpack_sum']['frac']})", file=sys.stderr, flush=True)
    return out


# ---------------------------------------------------------------------------
# Capacity-factor variant (token dropping) on the timed workload
# ---------------------------------------------------------------------------

def capacity_bench(bench, steps, warmup, factors=(1.0, 1.25)):
    """moe_layer_capacity on the bench's own layer and batch: C =
    ceil(cf * T * k / E) pairs per expert; the hottest expert is capped, at
    the price of the dropped (token, expert) pairs.  Each factor in the packed
    layout and in the padded one (fixed blocks of C rows per expert; payload =
    kept pairs over those rows).  Graph-replayed times beside the dropless
    time of the same batch."""
    import torch
    M, cfg, T = bench.M, bench.cfg, bench.T
    if cfg.dtype != "bf16":
        return None
    dropped = torch.zeros((4,), dtype=torch.int32, device="cuda")
    saved = bench.layer_fn
    out = []
    try:
        for cf in factors:
            C = int(math.ceil(cf * T * cfg.k / cfg.E))
            for padded in (0, 1):
                ws_p = M.layer_workspace(bench.layers[0][0], T, capacity=C, padded=1) \
                    if padded else None

                def fn(d, T_, x, y, ws, nb, dbg=None, C=C, padded=padded, ws_p=ws_p):
                    if ws_p is not None:
                        ws, nb = ws_p, ws_p.numel()
                    M.moe_layer_capacity(d, T_, C, padded, x, y, ws, nb, dbg, dropped)

                bench.layer_fn = fn
                bench.step(0)
                torch.cuda.synchronize()
                n_drop = int(dropped[0].item())
                ms = bench.timed_graph(steps, warmup)
                kept = T * cfg.k - n_drop
                rec = dict(capacity_factor=cf, capacity=C,
                           layout="padded" if padded else "packed", dropped_pairs=n_drop,
                           dropped_frac=round(n_drop / (T * cfg.k), 4), ms=round(ms, 4),
                           tokens_per_s=round(T / (ms * 1e-3), 1))
                if padded:
                    rec["payload_frac"] = round(kept / (cfg.E_loc * C), 4)
                out.append(rec)
                print(f"# capacity cf={cf} {rec['layout']}: C={C}, dropped "
                      f"{n_drop / (T * cfg.k):.3f} of the pairs, {ms:.4f} ms", file=sys.stderr,
                      flush=True)
                del ws_p
    finally:
        bench.layer_fn = saved
    return out


# ---------------------------------------------------------------------------
# EP <-> TP weight reshard, the data movement on one rank
# ---------------------------------------------------------------------------

def reshard_bench(steps, warmup, P=8):
    """moe_reshard_ep_to_tp_pack and moe_reshard_tp_to_ep_interleave on one
    rank's share of the Qwen3-235B-A22B-shaped layer at P = 8 (16 whole
    experts, I = 1536, H = 4096, bf16), timed by HIP-graph replay.
    Algorithmic bytes: every weight byte of the share read once and written
    once."""
    import torch
    import mixture_experts_layer_amd as M
    import workloads as W
    cfg = W.CONFIGS["qwen3_ep_all128"]
    n, I, H = cfg.E // P, cfg.I, cfg.H
    g = torch.Generator(device="cuda").manual_seed(0)
    w13 = torch.randn((n, 2 * I, H), generator=g, device="cuda").to(torch.bfloat16)
    w2 = torch.randn((n, H, I), generator=g, device="cuda").to(torch.bfloat16)
    c13 = torch.empty((P, n, 2 * I // P, H), dtype=torch.bfloat16, device="cuda")
    c2 = torch.empty((P, n, H, I // P), dtype=torch.bfloat16, device="cuda")
    o13, o2 = torch.empty_like(w13), torch.empty_like(w2)
    dt = M.dtype_code(w13)
    nbytes = 2 * (w13.numel() + w2.numel()) * 2
    res = dict(workload="qwen3_235b_a22b expert weights, one of %d ranks (%d experts, I=%d, H=%d)"
               % (P, n, I, H), weight_bytes=(w13.numel() + w2.numel()) * 2)
    for name, fn in (
            ("ep_to_tp_pack", lambda: M.moe_reshard_ep_to_tp_pack(w13, w2, n, I, H, P, dt, c13, c2)),
            ("tp_to_ep_interleave",
             lambda: M.moe_reshard_tp_to_ep_interleave(c13, c2, n, I, H, P, dt, o13, o2))):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(4):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // 4)
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / (reps * 4)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = dict(ms=round(ms, 4), algorithmic_bytes=int(nbytes), achieved_GBs=round(gbs, 1),
                         peak_GBs=HBM_PEAK_GBS, frac=round(gbs / HBM_PEAK_GBS, 4))
    torch.cuda.synchronize()
    assert torch.equal(o13, w13) and torch.equal(o2, w2), "reshard round trip changed the weights"
    print(f"# reshard: pack {res['ep_to_tp_pack']['ms']} ms ({res['ep_to_tp_pack']['frac']}), "
          f"interleave {res['tp_to_ep_interleave']['ms']} ms ({res['tp_to_ep_interleave']['frac']})",
          file=sys.stderr, flush=True)
    return res


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)
# ---------------------------------------------------------------------------

def cpu_baseline(bench, n_sample, min_seconds):
    import numpy as np
    import torch
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    L, cfg = bench.L, bench.cfg
    W = bench.W
    T = bench.T
    n = T if n_sample is None else min(n_sample, T)
    idx = W.sample_rows(T, n, seed=1).numpy()
    f = lambda t: None if t is None else t.float().cpu().numpy()
    x = f(L.x[:T])[idx]
    w_r = f(L.w_r)
    lb = f(L.logit_bias)
    sb = f(L.sel_bias)
    # host copies of the weights stay in their storage dtype; the oracle's
    # per-expert widening to float32 is inside the timed region
    w13_h = bench.layers[0][1].cpu()
    w2_h = bench.layers[0][2].cpu()

    class V:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, e):
            return self.t[e].float().numpy()

    kw = {}
    if cfg.I_shared:
        kw = dict(w13_shared=f(L.w13_shared), w2_shared=f(L.w2_shared))
    passes, dt = 0, 0.0
    while passes == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        O.moe_layer(x, w_r, V(w13_h), V(w2_h), cfg.k, cfg.mode, logit_bias=lb, sel_bias=sb,
                    dtype=np.float32, **kw)
        dt += time.perf_counter() - t0
        passes += 1
    what = "all" if n == T else f"{n} (seeded subset) of the"
    return dict(value=round(passes * n / dt, 2), unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"{passes} pass(es) over {what} {T} tokens, float32 numpy oracle, "
                       f"per-expert bf16->fp32 widening inside the timed region; {dt:.1f} s")


# ---------------------------------------------------------------------------
# HBM traffic of the dominant kernel, from the committed counter summary
# ---------------------------------------------------------------------------

def _csrc(*names):
    return [os.path.join(ROOT, "mixture_experts_layer_amd", "csrc", f) for f in names]


# Counter summaries of the kernels a roofline entry is quoted on, each with
# every source that kernel is compiled from.
TRAFFIC_PROFILES = {
    "gemm_gate_up": (os.path.join(ROOT, "profiles", "qwen3_ep_all128_T8192_gemm_gate_up_traffic.md"),
                     _csrc("ffn.hip", "moe_device.h", "moe_kernels.h")),
    "decode": (os.path.join(ROOT, "profiles", "qwen3_tp8_rank0_T1_decode_traffic.md"),
               _csrc("decode.hip", "moe_gate.h", "moe_router.h", "moe_device.h", "moe_kernels.h")),
}


def kernel_source_sha256(kernel="gemm_gate_up"):
    import hashlib
    h = hashlib.sha256()
    for path in TRAFFIC_PROFILES[kernel][1]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(kernel, workload, T):
    """Bytes per launch of `kernel` measured with FETCH_SIZE and WRITE_SIZE
    (scaled by the copy-kernel calibration), if its summary was taken on this
    workload and on the kernel source as it is now."""
    try:
        with open(TRAFFIC_PROFILES[kernel][0]) as f:
            line = next(l for l in f if l.startswith("traffic_json: "))
        rec = json.loads(line[len("traffic_json: "):])
    except (OSError, StopIteration, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("T") != T:
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha256(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_probe():
    import torch
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe": "torch.neg float32", "read_bytes": 1 << 30,
                      "write_bytes": 1 << 30, "dispatches": 3}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: the library computes one GPU's share of the layer, and the exchanges "
              "between GPUs are not part of it.", flush=True)
        sys.exit(2)
    import torch
    import workloads as W
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe()
        return
    cfg = W.CONFIGS[args.workload]
    T = args.T or cfg.T_max

    bench = Bench(args.workload, T, args.copies, args.path)
    counts = bench.counts()
    work = layer_work(cfg, T, counts, bench.I_loc, bench.elt)
    bench.size_rotation(work)
    ms, split = bench.timed_eager(args.steps, args.warmup)
    path = bench.path_of(T)
    l_bound, t_roof_ms, l_frac = layer_roof_frac(cfg, work, ms)
    ms_graph = bench.timed_graph(args.steps, args.warmup)
    if path == "decode":
        # One launch covers the whole layer.  Events around a single launch add
        # a few microseconds to a kernel of about thirty; the events bracketing
        # the graph replays (one launch per weight copy, back to back on this
        # stream) add only the dispatch gap between launches.
        t_k = bench.graph_event_ms
        roof = decode_roofline_entry(cfg, work, t_k)
        roof["kernel"] = "single-launch decode kernel (graph-replayed launches, events on the launch stream)"
        roof["traffic"] = committed_traffic("decode", WORKLOAD_NAMES[args.workload], T)
        roof["algorithmic_bytes"] = work["b_alg"]
        roof["avg_launch_ms"] = round(t_k, 4)
    else:
        roof = roofline_entry(cfg, work, split["gemm_gate_up"])
        roof["kernel"] = "grouped gate/up GEMM + SwiGLU (moe_layer stage events 1 -> 2)"
        roof["traffic"] = committed_traffic("gemm_gate_up", WORKLOAD_NAMES[args.workload], T)
        roof["algorithmic_bytes"] = work["g1_bytes"]
        roof["avg_launch_ms"] = round(split["gemm_gate_up"], 4)

    capacity = None
    if not args.no_capacity and path == "staged":
        capacity = dict(dropless_ms_graph=round(ms_graph, 4),
                        variants=capacity_bench(bench, args.steps, args.warmup))

    sweep = []
    if not args.no_sweep:
        for name in [s for s in args.sweep_workloads.split(",") if s]:
            c2 = W.CONFIGS[name]
            Ts = [T2 for T2 in c2.T_list if not (name == args.workload and T2 == T)]
            if not Ts:
                continue
            # the timed bench serves its own workload's sweep if it holds enough tokens
            b2 = bench if name == args.workload and bench.T_max >= max(Ts) else \
                Bench(name, max(Ts), None, args.path)
            for T2 in Ts:
                b2.set_T(T2)
                c2counts = b2.counts()
                w2k = layer_work(c2, T2, c2counts, b2.I_loc, b2.elt)
                n_copies = b2.size_rotation(w2k)
                ms2 = b2.timed_graph(max(args.steps, 20), args.warmup)
                bd, tr, fr = layer_roof_frac(c2, w2k, ms2)
                sweep.append(dict(workload=WORKLOAD_NAMES[name], T=T2, path=b2.path_of(T2),
                                  ms=round(ms2, 4),
                                  tokens_per_s=round(T2 / (ms2 * 1e-3), 1), bound=bd,
                                  roofline_ms=round(tr, 4), frac=round(fr, 4),
                                  weight_copies=n_copies,
                                  rotation_touched_bytes=int(
                                      n_copies * (w2k["b_alg"] - 2 * b2.elt * T2 * c2.H)),
                                  routing=routing_shape(c2counts, T2, c2.k, c2.E)))
                print(f"# sweep {name} T={T2}: {ms2:.4f} ms, {fr:.3f} of roofline ({bd})",
                      file=sys.stderr, flush=True)
            if b2 is not bench:
                del b2
                torch.cuda.empty_cache()
            bench.set_T(T)
            bench.size_rotation(work)

    dispatch = None
    if not args.no_dispatch:
        dispatch = dispatch_bench(max(args.steps, 20), args.warmup)

    reshard = None
    if not args.no_reshard:
        reshard = reshard_bench(max(args.steps, 20), args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(bench, args.cpu_sample, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "T": T, "H": cfg.H,
                   "I_loc": bench.I_loc, "E": cfg.E, "k": cfg.k, "gating_mode": cfg.mode,
                   "I_shared": cfg.I_shared, "weight_copies": bench.copies,
                   "rotation_touched_bytes": int(bench.copies * (work["b_alg"] - 2 * bench.elt * T
                                                                 * cfg.H)),
                   "parallelism": "single-gpu share", "entry_point": LAYER_FN[args.path],
                "path": path},
        "roofline": roof,
        "layer_roofline": {"bound": l_bound, "t_roof_ms": round(t_roof_ms, 4),
                           "frac": round(l_frac, 4), "b_alg_bytes": work["b_alg"],
                           "f_alg_flops": work["f_alg"]},
        "ms_per_step_graph": round(ms_graph, 4),
        "stage_ms": {k2: round(v, 4) for k2, v in split.items()},
        "routing": routing_shape(counts, T, cfg.k, cfg.E),
        "sweep": sweep,
        "capacity": capacity,
        "dispatch": dispatch,
        "reshard": reshard,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
