"""Shared test plumbing: run the HIP path through the C ABI, run the oracle on
the same inputs, and compare per the parity protocol.

Parity protocol (GPU vs oracle):
  1. GPU float32 logits vs the oracle's float64 logits: |d| <= 1e-5 * max|s|.
  2. The oracle's gating runs on the GPU's float32 logits (mode 3 adds the
     float32 selection bias in float32 on both sides): ids, counts, offsets,
     src_token and dst_row must match exactly.
  3. The oracle's experts and combine (float64) on those ids give the
     reference output: max|d| / max|ref| <= 1e-2 for bf16 layers, 1e-5 for
     float32 layers.
"""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_layer_amd as M
import workloads as W
from oracle import moe_oracle as O

TOL = {"bf16": 1e-2, "f32": 1e-5}


def to_np(t):
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


class ExpertView:
    """Index a [E, ...] device tensor expert by expert as float32 numpy arrays
    (bf16 widens exactly), so the oracle touches only the experts it uses."""

    def __init__(self, t):
        self.t = t

    def __len__(self):
        return self.t.shape[0]

    def __getitem__(self, e):
        return to_np(self.t[e])


class OracleShare:
    """The oracle's own cut of one GPU's share from the FULL expert tensors:
    local expert i is expert e_begin + i, and a tensor-parallel share goes
    through oracle.tp_shard.  Independent of workloads.share_weights, which
    prepares the GPU's copy."""

    def __init__(self, w13_full, w2_full, e_begin=0, tp_P=1, tp_rank=0):
        self.w13, self.w2 = w13_full, w2_full
        self.e_begin, self.P, self.r = e_begin, tp_P, tp_rank
        self._cache = {}

    def get(self, i):
        if i not in self._cache:
            if len(self._cache) > 2:
                self._cache.clear()
            e = self.e_begin + i
            a13, a2 = to_np(self.w13[e])[None], to_np(self.w2[e])[None]
            if self.P > 1:
                a13, a2 = O.tp_shard(a13, a2, self.r, self.P)
            self._cache[i] = (a13[0], a2[0])
        return self._cache[i]

    def view(self, which):
        share = self

        class _V:
            def __getitem__(self, i):
                return share.get(i)[which]
        return _V()


def ws_tensor(nbytes, device="cuda"):
    # zeroed: a layer workspace starts with the decode path's sync block
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


LAYER_FNS = {"auto": "moe_layer", "staged": "moe_layer_staged", "decode": "moe_layer_decode"}


class GpuLayer:
    """One layer share on the GPU: weights, descriptor and workspace for T_max."""

    def __init__(self, L: W.LayerInputs, tp_P=1, tp_rank=0, e_begin=0, e_end=None, T_max=None):
        cfg = L.cfg
        self.L = L
        self.E = L.w_r.shape[0]
        self.H = L.w_r.shape[1]
        self.k = cfg.k
        self.mode = cfg.mode
        self.e_begin = e_begin
        self.e_end = self.E if e_end is None else e_end
        self.tp_P, self.tp_rank = tp_P, tp_rank
        self.w13, self.w2 = W.share_weights(L.w13, L.w2, tp_P, tp_rank, e_begin, self.e_end)
        self.I_loc = self.w13.shape[1] // 2
        self.I_shared = 0 if L.w13_shared is None else L.w13_shared.shape[0] // 2
        self.dt = M.dtype_code(L.x)
        self.desc = M.layer_desc(self.H, self.E, self.k, self.I_loc, self.mode, self.dt, L.w_r,
                                 self.w13, self.w2, e_begin=self.e_begin, e_end=self.e_end,
                                 I_shared=self.I_shared, w13_shared=L.w13_shared,
                                 w2_shared=L.w2_shared, logit_bias=L.logit_bias,
                                 sel_bias=L.sel_bias)
        T_max = T_max or L.x.shape[0]
        self.ws_bytes = M.moe_layer_workspace_size(self.desc, T_max)
        assert self.ws_bytes > 0
        self.ws = ws_tensor(self.ws_bytes)

    def run(self, T, x=None, debug=True, path="auto"):
        x = self.L.x[:T] if x is None else x
        dev = x.device
        E_loc = self.e_end - self.e_begin
        y = torch.empty((T, self.H), dtype=x.dtype, device=dev)
        out = dict(y=y)
        dbg = None
        if debug:
            out.update(
                logits=torch.empty((T, self.E), dtype=torch.float32, device=dev),
                ids=torch.empty((T, self.k), dtype=torch.int32, device=dev),
                w=torch.empty((T, self.k), dtype=torch.float32, device=dev),
                counts=torch.empty((E_loc,), dtype=torch.int32, device=dev),
                offsets=torch.empty((E_loc + 1,), dtype=torch.int32, device=dev),
                src_token=torch.empty((max(T * self.k, 1),), dtype=torch.int32, device=dev),
                dst_row=torch.empty((T, self.k), dtype=torch.int32, device=dev))
            dbg = M.debug_out(out["logits"], out["ids"], out["w"], out["counts"], out["offsets"],
                              out["src_token"], out["dst_row"])
        getattr(M, LAYER_FNS[path])(self.desc, T, x, y, self.ws, self.ws_bytes, dbg)
        self.last_path = path if path != "auto" else M.moe_layer_path(self.desc, T)
        return out

    def sync_error(self):
        """The decode path's error word (bytes 4..7 of the workspace)."""
        return int(self.ws[4:8].view(torch.int32).item())


def check_layer(gl: GpuLayer, out, T, sample=None, check_rows=True):
    """Apply the parity protocol to one moe_layer run.  `sample`: token indices
    whose outputs are checked (None = all), or a function of the run's outputs
    returning them (called once the routing metadata has matched); routing
    metadata is always checked for the whole batch.  Returns a dict of
    measured errors."""
    torch.cuda.synchronize()
    if getattr(gl, "last_path", None) == "decode":
        # no wait of the single-launch path ran out (raises MoEError otherwise)
        M.moe_layer_status(gl.ws, gl.ws_bytes)
    L, cfg = gl.L, gl.L.cfg
    x = to_np(L.x[:T])
    logits_gpu = to_np(out["logits"])
    w_r = to_np(L.w_r)
    lb = to_np(L.logit_bias)
    sb = to_np(L.sel_bias)
    res = {}
    # 1. logits
    s_ref = O.router_logits(x, w_r, lb)
    err = np.abs(logits_gpu.astype(np.float64) - s_ref).max() / max(np.abs(s_ref).max(), 1e-30)
    res["logits_rel"] = float(err)
    assert err <= 1e-5, f"logits rel err {err}"
    # 2. gating + permutation on the GPU's float32 logits
    ids_ref, w_ref = O.route(logits_gpu, gl.k, gl.mode, sb)
    ids_gpu = to_np(out["ids"])
    assert np.array_equal(ids_gpu, ids_ref), "top-k ids differ"
    w_gpu = to_np(out["w"])
    res["w_abs"] = float(np.abs(w_gpu - w_ref).max())
    assert res["w_abs"] <= 2e-6, f"gate weights differ by {res['w_abs']}"
    counts, offsets, src, dst = O.permute(ids_ref, gl.e_begin, gl.e_end)
    assert np.array_equal(to_np(out["counts"]), counts), "counts differ"
    assert np.array_equal(to_np(out["offsets"]), offsets), "offsets differ"
    rows = int(offsets[-1])
    assert np.array_equal(to_np(out["src_token"])[:rows], src), "src_token differs"
    assert np.array_equal(to_np(out["dst_row"]), dst), "dst_row differs"
    if not check_rows:
        return res
    # 3. outputs
    if callable(sample):
        sample = sample(out)
    idx = np.arange(T) if sample is None else np.asarray(sample)
    res["tokens_checked"] = int(len(idx))
    share = OracleShare(L.w13, L.w2, gl.e_begin, gl.tp_P, gl.tp_rank)
    w13, w2 = share.view(0), share.view(1)
    kw = {}
    if gl.I_shared:
        kw = dict(w13_shared=to_np(L.w13_shared), w2_shared=to_np(L.w2_shared))
    y_ref, _ = O.moe_layer(x[idx], None, w13, w2, gl.k, gl.mode, sel_bias=sb,
                           e_begin=gl.e_begin, e_end=gl.e_end, logits=logits_gpu[idx], **kw)
    y_gpu = to_np(out["y"])[idx].astype(np.float64)
    scale = max(np.abs(y_ref).max(), 1e-30)
    res["y_rel"] = float(np.abs(y_gpu - y_ref).max() / scale)
    tol = TOL[cfg.dtype]
    assert res["y_rel"] <= tol, f"layer output rel err {res['y_rel']} > {tol}"
    return res


def boundary_sample(T, n_random, seed, tiles=(128, 256)):
    """A function of a run's outputs giving the tokens whose outputs a
    full-size case checks: every token whose copy sits on an expert
    segment's first or last row, on the first row of its last row tile or on
    the last row before it (for each GEMM row tile in `tiles`: the ragged
    tails and the tile boundaries), plus `n_random` seeded tokens.  Exact
    for a dropless layer: a token's output depends on that token alone."""
    def pick(out):
        offsets = to_np(out["offsets"]).astype(np.int64)
        src = to_np(out["src_token"]).astype(np.int64)
        toks = set(W.sample_rows(T, n_random, seed=seed).tolist())
        for e in range(len(offsets) - 1):
            r0, r1 = int(offsets[e]), int(offsets[e + 1])
            if r1 <= r0:
                continue
            rows = {r0, r1 - 1}
            for bm in tiles:
                last = r0 + bm * ((r1 - 1 - r0) // bm)
                rows.update((last, max(last - 1, r0)))
            toks.update(int(src[r]) for r in rows)
        return np.array(sorted(toks), dtype=np.int64)
    return pick
