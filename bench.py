"""Benchmark of the Veda block-sparse attention layer on one MI355X.

One step = one attention layer through the whole hot path on one batch of
resident synthetic input: permute Q, K (rows) and V (tile-transposed) with the
tile pooling fused in, project and score tile pairs, select blocks, and run
block-sparse attention whose epilogue writes O back in natural token order
(plus, for the packed workload, the dense LSE and the block heat over all
blocks, by default in the same pass as the attention, the oracle mask
selected on the heat and the attention mass of the predicted and the oracle
mask).  Four seeded input
sets rotate across steps, so each call sees a new block pattern.

Prints one JSON line.  value = attention FLOP over computed blocks / layer
time (TFLOP/s); ms_per_step = ms per layer; roofline = the attention kernel
alone, timed with HIP events on the stream it runs on.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

import veda_workloads as wl

METRIC = "block-sparse attn TFLOP/s over computed blocks + ms/layer at 90% sparsity"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=4,
                    help="workload index 1..5 (default 4: the long clip, the largest workload that fits one GPU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (known bytes) to scale HBM counters")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="rough budget of the oracle sample")
    ap.add_argument("--separate-heat", action="store_true",
                    help="packed workload: the attention and the dense LSE + heat as two calls instead of "
                         "veda_attn_fwd_lse_heat")
    ap.add_argument("--q-copy", action="store_true",
                    help="write the permuted copy of Q in the layer and have the attention read it, instead of "
                         "gathering Q's rows from the natural layout in the attention kernel")
    ap.add_argument("--backward", action="store_true",
                    help="also time the block-sparse backward (transposed lists, dK/dV and dQ) of the same layer")
    ap.add_argument("--search", action="store_true",
                    help="also time the tile-plan search on the 8x32x32 grid (16 heads, D 128, 10%% keep, "
                         "5 candidate shapes, 3 samples of one layer) and report it")
    ap.add_argument("--traffic-json", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "profiles", "traffic.json"))
    return ap.parse_args()


class Layer:
    """Device buffers and the calls of one attention layer."""

    def __init__(self, w, inputs, vb, q_copy=False, separate_heat=False):
        self.w, self.vb = w, vb
        # with the heat: the attention and the dense LSE + heat in one call
        # (veda_attn_fwd_lse_heat: no block's scores computed twice) unless
        # separate_heat
        self.split_heat = bool(w.with_heat) and not separate_heat
        # q_copy: the permutation also writes the permuted copy of Q and the
        # attention reads it; by default the attention gathers Q's rows from
        # the natural [N, H, D] layout and no copy of Q is written
        self.q_copy = q_copy
        self.plan = vb.Plan.from_workload(w)
        p = self.plan
        dev = "cuda"
        self.sets = [{k: t.to(dev) for k, t in inp.items()} for inp in inputs]
        self.qp, self.kp, self.vt = p.empty_perm(), p.empty_perm(), p.empty_vt()
        self.scores = torch.empty(p.info["total_pairs"], dtype=torch.float32, device=dev)
        self.ws = p.empty_workspace()
        self.row_ptr = torch.empty(p.T + 1, dtype=torch.int32, device=dev)
        self.col = torch.empty(p.info["nnz"], dtype=torch.int32, device=dev)
        self.lse = torch.empty(p.R, dtype=torch.float32, device=dev)
        self.o_nat = torch.empty((w.num_tokens, w.num_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        self.dense = None
        if w.with_heat:
            self.dense = vb.Plan.from_workload(w, budget_mode=wl.ALL_BLOCKS)
            self.d_row_ptr = torch.empty(p.T + 1, dtype=torch.int32, device=dev)
            self.d_col = torch.empty(self.dense.info["nnz"], dtype=torch.int32, device=dev)
            self.d_lse = torch.empty(p.R, dtype=torch.float32, device=dev)
            self.heat = torch.empty(p.info["total_pairs"], dtype=torch.float32, device=dev)
            self.heat_ws = torch.empty(self.dense.info["heat_workspace_bytes"] // 4, dtype=torch.float32,
                                       device=dev)
            # oracle mask (selection on the heat) and the attention mass of both masks
            self.o_row_ptr = torch.empty(p.T + 1, dtype=torch.int32, device=dev)
            self.o_col = torch.empty(p.info["nnz"], dtype=torch.int32, device=dev)
            self.m_pred = torch.empty(w.num_heads, dtype=torch.float64, device=dev)
            self.m_orc = torch.empty(w.num_heads, dtype=torch.float64, device=dev)
        self.attn_events = []
        self.perm_events = []

    def q_of(self, x):
        """The Q operand of the attention calls and its layout."""
        if self.q_copy:
            return self.qp, self.vb.VEDA_LAYOUT_PERMUTED
        return x["q"], self.vb.VEDA_LAYOUT_NATURAL

    def step(self, s, time_attn=False):
        vb, p, w = self.vb, self.plan, self.w
        x = self.sets[s % len(self.sets)]
        if time_attn:
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record()
        p.permute_qkv(x["q"], x["k"], x["v"], self.qp if self.q_copy else None, self.kp, self.vt, self.ws)
        if time_attn:
            g1.record()
            self.perm_events.append((g0, g1))
        p.score_pooled(x["w_q"], x["w_k"], self.scores, self.ws)
        p.select(self.scores, self.row_ptr, self.col)
        q, ql = self.q_of(x)
        if self.split_heat:
            d = self.dense
            d.select(self.scores, self.d_row_ptr, self.d_col)
        if time_attn:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        if self.split_heat:
            # the attention of the predicted mask, the dense LSE and the block heat in one pass
            p.attention_lse_heat(d, q, self.kp, self.vt, self.row_ptr, self.col, self.d_row_ptr, self.d_col,
                                 w.softmax_scale, self.o_nat, self.lse, self.d_lse, self.heat, self.heat_ws,
                                 o_layout=vb.VEDA_LAYOUT_NATURAL, q_layout=ql)
        else:
            p.attention(q, self.kp, self.vt, self.row_ptr, self.col, w.softmax_scale, self.o_nat, self.lse,
                        o_layout=vb.VEDA_LAYOUT_NATURAL, q_layout=ql)
        if time_attn:
            e1.record()
            self.attn_events.append((e0, e1))
        if self.dense is not None:
            d = self.dense
            if not self.split_heat:
                d.select(self.scores, self.d_row_ptr, self.d_col)
                # the dense LSE and the block heat in one pass over all blocks
                d.lse_heat(q, self.kp, self.d_row_ptr, self.d_col, w.softmax_scale, self.d_lse, self.heat,
                           self.heat_ws, q_layout=ql)
            p.select(self.heat, self.o_row_ptr, self.o_col)
            p.mask_mass(self.heat, self.row_ptr, self.col, self.m_pred)
            p.mask_mass(self.heat, self.o_row_ptr, self.o_col, self.m_orc)


def cpu_baseline(w, inp, budget_s, total_blocks):
    """The oracle on a bounded sample of the same workload, timed stage by
    stage on the host: for heads 0, 1, ... (one-head oracle plans, which give
    exactly that head's part of the all-heads oracle) the permutation of Q, K
    and V, the pooling, projection and scores, the selection, the attention of
    query tiles in ascending order and the inverse permutation of O, until
    about budget_s seconds are spent (at least one head's front stages and one
    query tile).  Each stage is extrapolated to the whole layer: the front
    stages and the inverse permutation by heads, the attention by computed
    blocks.  value = the layer's attention FLOP over computed blocks / the
    extrapolated layer time, the metric's unit."""
    from oracle import veda_oracle as vo
    threads = torch.get_num_threads()
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max(blas) if blas else threads
    except Exception:
        pass
    per_block = 4.0 * 128 * 128 * w.head_dim
    qn = inp["q"].to(torch.float64).numpy()
    kn = inp["k"].to(torch.float64).numpy()
    vn = inp["v"].to(torch.float64).numpy()
    t = {"permute_qkv": 0.0, "pool": 0.0, "project_score": 0.0, "select": 0.0, "attention": 0.0,
         "unpermute_o": 0.0}
    heads_front, tiles_attn, blocks_attn, heads_attn_whole = 0, 0, 0, 0
    spent = 0.0
    clock = time.perf_counter
    for h in range(w.num_heads):
        sub = vo.Plan(w.segments, 1, w.head_dim, [w.tile_shapes[h]], w.budget_mode, w.keep_num, w.keep_den,
                      w.fixed_k)
        c0 = clock()
        qp = vo.permute_forward(sub, qn[:, h:h + 1])
        kp = vo.permute_forward(sub, kn[:, h:h + 1])
        vp = vo.permute_forward(sub, vn[:, h:h + 1])
        c1 = clock()
        fq, fk = vo.pool_tiles(sub, qp), vo.pool_tiles(sub, kp)
        c2 = clock()
        qh = vo.project(sub, fq, inp["w_q"].numpy()[h:h + 1])
        kh = vo.project(sub, fk, inp["w_k"].numpy()[h:h + 1])
        scores = vo.score_pairs(sub, qh, kh)
        c3 = clock()
        sel = vo.select_blocks(sub, scores)
        c4 = clock()
        t["permute_qkv"] += c1 - c0
        t["pool"] += c2 - c1
        t["project_score"] += c3 - c2
        t["select"] += c4 - c3
        heads_front += 1
        spent += c4 - c0
        n = sub.heads[0].num_tiles
        done = 0
        for i in range(n):
            a0 = clock()
            vo.attention_row_tile(sub, 0, i, qp, kp, vp, sel[0][i], w.softmax_scale)
            dt = clock() - a0
            t["attention"] += dt
            spent += dt
            tiles_attn += 1
            blocks_attn += len(sel[0][i])
            done += 1
            if spent >= budget_s:
                break
        if done == n:
            heads_attn_whole += 1
        u0 = clock()
        o_perm = np.zeros((sub.total_rows, w.head_dim))
        vo.permute_inverse(sub, o_perm)
        du = clock() - u0
        t["unpermute_o"] += du
        spent += du
        if spent >= budget_s:
            break
    H = w.num_heads
    layer_s = {k: v * H / heads_front for k, v in t.items() if k != "attention"}
    layer_s["attention"] = t["attention"] * total_blocks / blocks_attn
    heat_note = ""
    if w.with_heat:
        # the dense LSE (the oracle's attention over every key tile of the
        # row; it also forms an O that is not used) and the block heat of
        # query tiles 0, 1, ... of head 0, about a quarter of budget_s,
        # extrapolated by query tiles (every head of the packed workload has
        # the same tile count)
        sub = vo.Plan(w.segments, 1, w.head_dim, [w.tile_shapes[0]], wl.ALL_BLOCKS, 1, 1, 0)
        qp, kp = vo.permute_forward(sub, qn[:, :1]), vo.permute_forward(sub, kn[:, :1])
        n = sub.heads[0].num_tiles
        L = np.full(sub.total_rows, np.nan)
        rows = []
        d0 = clock()
        for i in range(n):
            _, Li = vo.attention_row_tile(sub, 0, i, qp, kp, kp, range(n), w.softmax_scale)
            L[128 * i: 128 * i + sub.heads[0].tiles[i].valid] = Li
            rows.append(i)
            if clock() - d0 >= budget_s / 4:
                break
        d1 = clock()
        vo.block_heat(sub, qp, kp, L, w.softmax_scale, rows=rows)
        d2 = clock()
        t["dense_lse"], t["heat"] = d1 - d0, d2 - d1
        spent += d2 - d0
        total_tiles = n * H
        layer_s["dense_lse"] = t["dense_lse"] * total_tiles / len(rows)
        layer_s["heat"] = t["heat"] * total_tiles / len(rows)
        heat_note = "; the dense LSE and the heat of %d query tiles of head 0, extrapolated by query tiles" % len(rows)
    layer_ms = 1e3 * sum(layer_s.values())
    return {"value": total_blocks * per_block / (layer_ms * 1e-3) / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "fp64 numpy oracle, %.1f s on the host: front stages (permute Q/K/V, pool, project+score, "
                      "select) and the inverse permutation of heads 0..%d of %d, attention of %d query tiles "
                      "(%d blocks of %d in the layer; %d whole heads); each stage extrapolated to the layer "
                      "(front stages by heads, attention by blocks)%s" % (spent, heads_front - 1, H, tiles_attn,
                                                                          blocks_attn, total_blocks,
                                                                          heads_attn_whole, heat_note),
            "ms_per_layer_extrapolated": round(layer_ms, 1),
            "stage_ms_sample": {k: round(1e3 * v, 1) for k, v in t.items()},
            "stage_ms_per_layer_extrapolated": {k: round(1e3 * v, 1) for k, v in layer_s.items()},
            "attention_tflops": round(blocks_attn * per_block / t["attention"] / 1e12, 5),
            "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the Veda path shards by heads with no exchange, and the library "
              "has no multi-GPU path (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    from block_sparse_attention_10_amd import binding as vb
    ok, why = vb.veda_available(0)
    if not ok:
        print("libveda unavailable: " + why, file=sys.stderr)
        sys.exit(1)
    w = wl.workload(args.config)
    print("bench: generating inputs for %s" % w.describe(), file=sys.stderr, flush=True)
    inputs = [wl.make_inputs(w, seed=s) for s in wl.rotation_seeds(w)]
    layer = Layer(w, inputs, vb, q_copy=args.q_copy, separate_heat=args.separate_heat)
    p = layer.plan
    nnz = p.info["nnz"]
    flops_attn = 4.0 * 128 * 128 * w.head_dim * nnz
    # the timed kernels' work: the attention, plus with the split heat call the
    # dense QK^T products (2 * 128^2 * D per block of the all-blocks mask)
    flops_kernel = flops_attn
    if layer.split_heat:
        flops_kernel += 2.0 * 128 * 128 * w.head_dim * layer.dense.info["nnz"]
    print("bench: warmup %d, steps %d, nnz %d" % (args.warmup, args.steps, nnz), file=sys.stderr, flush=True)
    for s in range(args.warmup):
        layer.step(s)
    torch.cuda.synchronize()
    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)     # 1 GiB read + 1 GiB written per launch
        torch.cuda.synchronize()
        del a, b
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(args.steps):
        layer.step(args.warmup + s, time_attn=True)
    t1.record()
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in layer.attn_events]
    attn_avg = float(np.mean(attn_ms))
    valid_flops = valid_only_flops(layer)
    cold = attention_cold(layer, 5)
    perm = permute_rate(layer, w)
    gemm = gemm_reference()
    attn_tflops = flops_kernel / (attn_avg * 1e-3) / 1e12
    value = flops_attn / (ms_step * 1e-3) / 1e12
    traffic = None
    try:
        with open(args.traffic_json) as f:
            tj = json.load(f)
        key = ("attn_lse_heat_config%d" if layer.split_heat else "attn_fwd_config%d") % args.config
        if key in tj and tj[key].get("kernel_code_sha") == kernel_code_sha(vb.loaded_library(), w.head_dim):
            traffic = tj[key]["bytes_per_launch"]
    except (OSError, ValueError, RuntimeError):
        pass
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, 4 rotating input sets)",
        "config": {"workload": "config %d %s" % (args.config, w.describe()), "tokens": w.num_tokens,
                   "heads": w.num_heads, "head_dim": w.head_dim, "nnz_blocks": nnz,
                   "block_density": round(nnz / p.info["total_pairs"], 4), "parallelism": "single GPU"},
        "attn_kernel": ("veda_attn_fwd_lse_heat: attn_mass_kernel + complement_kernel + rest_heat_kernel (the "
                        "attention and the dense LSE + heat; its work counts the dense QK^T products too)"
                        if layer.split_heat else "attn_fwd_kernel"),
        "attn_kernel_ms": round(attn_avg, 4), "attn_kernel_tflops": round(attn_tflops, 2),
        "attn_kernel_code_sha": _code_sha_or_none(vb.loaded_library(), w.head_dim),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "attn_kernel_calls": {"n": len(attn_ms), "median_ms": round(float(np.median(attn_ms)), 4),
                              "min_ms": round(float(np.min(attn_ms)), 4),
                              "p90_ms": round(float(np.percentile(attn_ms, 90)), 4)},
        "attn_valid_only_tflops": None if layer.split_heat else round(valid_flops / (attn_avg * 1e-3) / 1e12, 2),
        "attn_cold_cache": cold,
        "permute_qkv": perm,
        "q_operand": "permuted copy written by the permutation" if args.q_copy else
                     "natural [N, H, D] rows gathered by the attention kernel (no permuted copy of Q)",
        "bf16_gemm_reference": dict(gemm, attn_kernel_over_gemm=round(attn_tflops / gemm["tflops"], 4)),
        "library": vb.loaded_library(),
    }
    if layer.dense is not None:
        mp, mo = layer.m_pred.cpu().numpy(), layer.m_orc.cpu().numpy()
        out["mask_quality"] = {
            "oracle_mask_mass_mean": round(float(mo.mean()), 4),
            "predicted_mask_mass_mean": round(float(mp.mean()), 4),
            "recall_mean": round(float((mp / mo).mean()), 4), "recall_min": round(float((mp / mo).min()), 4),
            "note": "synthetic inputs and a random-init predictor; the pages' 0.63 / 0.71 come from real "
                    "activations"}
    if args.backward:
        out["backward"] = time_backward(layer, w, args.steps)
    if args.search:
        out["tile_plan_search"] = time_search()
    if not args.no_cpu_baseline:
        print("bench: oracle CPU baseline (~%.0f s)" % args.cpu_seconds, file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inputs[0], args.cpu_seconds, nnz)
    print(json.dumps(out), flush=True)


def valid_only_flops(layer):
    """Attention FLOP over valid (query, key) pairs only, 4 * nv(i) * nv(j) * D
    per computed block, for the mask of the last timed step (a secondary
    figure; the headline counts every computed block in full)."""
    vb, p, w = layer.vb, layer.plan, layer.w
    rp, col = layer.row_ptr.cpu().numpy(), layer.col.cpu().numpy()
    total, t0 = 0.0, 0
    for h in range(w.num_heads):
        nv = vb.veda_plan_copy_valid(p.handle, h).astype(np.float64)
        n = len(nv)
        for i in range(n):
            js = col[rp[t0 + i]:rp[t0 + i + 1]]
            total += nv[i] * float(nv[js].sum())
        t0 += n
    return 4.0 * w.head_dim * total


def permute_rate(layer, w):
    """The fused permutation + pooling of the timed steps (HIP events on the
    launch stream) against its algorithmic HBM bytes: every valid natural row
    of Q, K, V read once, every permuted row (padding included) written once,
    and the pooled features written; next to it, the rate of a plain 1 GiB
    device copy (1 GiB read + 1 GiB written) measured in the same run."""
    p = layer.plan
    ms = float(np.mean([a.elapsed_time(b) for a, b in layer.perm_events]))
    d = w.head_dim
    copies = 3 if layer.q_copy else 2      # permuted K and V^T (and Q with --q-copy)
    nbytes = (3 * w.num_tokens * w.num_heads * d * 2 + copies * p.R * d * 2 + 2 * p.T * 3 * d * 4)
    a = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_tbs = 2 * (1 << 30) / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12
    del a, b
    tbs = nbytes / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "bytes": nbytes, "tb_per_s": round(tbs, 3),
            "frac_of_hbm_peak": round(tbs * 1e3 / PEAK_HBM_GBS, 4), "copy_reference_tb_per_s": round(copy_tbs, 3),
            "frac_of_copy_rate": round(tbs / copy_tbs, 4)}


def gemm_reference(n=8192, reps=20):
    """Rate of the vendor bf16 GEMM (torch.matmul of two contiguous n x n
    matrices of N(0,1) values) in the same run: what the matrix cores sustain
    on random operands on this GPU, next to the nominal 2.5 PFLOP/s."""
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(5):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    return {"shape": "%dx%dx%d" % (n, n, n), "ms": round(ms, 4), "tflops": round(tf, 1),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def attention_cold(layer, n):
    """The attention call after a 1 GiB device write that evicts L2 and the
    last-level cache (mean of n calls, each on the next input set's mask)."""
    vb, p, w = layer.vb, layer.plan, layer.w
    scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    ms = []
    for s in range(n):
        layer.step(s)                      # this set's permutation and mask
        scrub.fill_(float(s))
        q, ql = layer.q_of(layer.sets[s % len(layer.sets)])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        p.attention(q, layer.kp, layer.vt, layer.row_ptr, layer.col, w.softmax_scale, layer.o_nat,
                    layer.lse, o_layout=vb.VEDA_LAYOUT_NATURAL, q_layout=ql)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del scrub
    note = "after a 1 GiB device write per call"
    if layer.split_heat:
        note += "; the separate attention call (veda_block_sparse_attn_fwd), not the fused heat pass"
    return {"n": n, "mean_ms": round(float(np.mean(ms)), 4), "note": note}


def time_backward(layer, w, steps):
    """The backward of the layer's last forward (same mask): transposed lists
    plus veda_block_sparse_attn_bwd, timed with HIP events; algorithmic work =
    2.5x the forward's (dV, dP, dK, dQ and the recomputed S: 10 * 128^2 * D
    flop per block)."""
    p, vb = layer.plan, layer.vb
    dev = "cuda"
    x = layer.sets[0]
    layer.step(0)                                          # K, V^T and the mask of input set 0
    p.permute(x["q"], layer.qp, vb.VEDA_PERMUTE_FORWARD)   # the backward takes permuted Q
    vp, dop, o = p.empty_perm(), p.empty_perm(), p.empty_perm()
    p.permute(x["v"], vp, vb.VEDA_PERMUTE_FORWARD)
    gen = torch.Generator().manual_seed(5)
    p.permute(torch.randn(x["v"].shape, generator=gen).to(torch.bfloat16).to(dev), dop, vb.VEDA_PERMUTE_FORWARD)
    p.attention(layer.qp, layer.kp, layer.vt, layer.row_ptr, layer.col, w.softmax_scale, o, layer.lse)
    col_ptr = torch.empty(p.T + 1, dtype=torch.int32, device=dev)
    row_idx = torch.empty(p.info["nnz"], dtype=torch.int32, device=dev)
    wt, wb = p.empty_bytes("transpose_workspace_bytes"), p.empty_bytes("bwd_workspace_bytes")
    dq, dk, dv = p.empty_perm(), p.empty_perm(), p.empty_perm()

    def run():
        p.transpose(layer.row_ptr, layer.col, col_ptr, row_idx, wt)
        p.backward(layer.qp, layer.kp, vp, o, dop, layer.lse, layer.row_ptr, layer.col, col_ptr, row_idx,
                   w.softmax_scale, dq, dk, dv, wb)
    for _ in range(3):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(3, min(steps, 20))
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flops = 10.0 * 128 * 128 * w.head_dim * p.info["nnz"]
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "tflops": round(tf, 2), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "flop_count": "10 * 128^2 * D per computed block (dV, dP, dK, dQ, recomputed S)",
            "includes": "transposed lists, per-row (lse, rowsum(dO*O)), key-tile dispatch order, dK/dV and dQ kernels"}


SEARCH_CANDIDATES = ((1, 8, 16), (2, 8, 8), (4, 4, 8), (2, 4, 16), (1, 16, 8))


def time_search():
    """Tile-plan search on one layer shaped like the 8x32x32 grid workload:
    three samples (fixed per-head length scales, new noise), five candidate
    shapes; one untimed run, then one timed run."""
    from block_sparse_attention_10_amd import search
    w = wl.Workload(98, "search_layer_8x32x32", (wl.Segment(wl.VIDEO3D, (8, 32, 32), 0),), 16, 128,
                    ((4, 4, 8),) * 16, wl.KEEP_RATIO, 1, 10)
    samples = []
    for s in range(3):
        x = wl.make_inputs(w, seed=700 + s, bias_seed=98)
        samples.append((x["q"].cuda(), x["k"].cuda(), x["v"].cuda()))
    args = (w.segments, w.num_heads, w.head_dim, SEARCH_CANDIDATES, w.budget_mode, w.keep_num, w.keep_den, 0,
            samples, w.softmax_scale)
    search.tile_plan_search(*args)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    err, choice = search.tile_plan_search(*args)
    ms = 1e3 * (time.perf_counter() - t0)
    counts = {str(SEARCH_CANDIDATES[c]): int((choice == c).sum()) for c in sorted(set(choice.tolist()))}
    return {"ms": round(ms, 2), "samples": 3, "candidates": len(SEARCH_CANDIDATES), "heads": w.num_heads,
            "grid": "8x32x32", "ms_per_sample_and_candidate": round(ms / (3 * len(SEARCH_CANDIDATES)), 3),
            "heads_per_chosen_shape": counts}


def _code_sha_or_none(lib_path, head_dim):
    try:
        return kernel_code_sha(lib_path, head_dim)
    except (OSError, ValueError, RuntimeError):
        return None


ATTN_SYMBOL = "_ZN4veda12_GLOBAL__N_115attn_fwd_kernelILi%dELb1EEEvNS_7DevPlanEPKtiS4_S4_PKiS6_fPtiPfPj"


def kernel_code_sha(lib_path, head_dim=128):
    """Hash of the attention kernel's machine code in the library that runs:
    the bytes of attn_fwd_kernel<D, true> in the gfx950 code object of the
    library's offload bundle, plus its kernel descriptor with the entry
    offset zeroed (the only field that depends on where the linker put the
    kernel).  Recorded traffic stays valid while this hash is unchanged,
    whatever else changes in the library."""
    import hashlib
    import struct
    with open(lib_path, "rb") as f:
        data = f.read()
    b0 = data.find(b"__CLANG_OFFLOAD_BUNDLE__")
    if b0 < 0:
        raise RuntimeError("no offload bundle in " + lib_path)
    n = struct.unpack_from("<Q", data, b0 + 24)[0]
    off, elf = b0 + 32, None
    for _ in range(n):
        o, size, tl = struct.unpack_from("<QQQ", data, off)
        triple = data[off + 24: off + 24 + tl]
        off += 24 + tl
        if triple.endswith(b"gfx950"):
            elf = data[b0 + o: b0 + o + size]
    if elf is None or elf[:4] != b"\x7fELF":
        raise RuntimeError("no gfx950 code object in " + lib_path)
    shoff = struct.unpack_from("<Q", elf, 0x28)[0]
    shentsize, shnum = struct.unpack_from("<HH", elf, 0x3A)
    # section headers: name, type, flags, addr, offset, size, link, info, align, entsize
    secs = [struct.unpack_from("<IIQQQQIIQQ", elf, shoff + k * shentsize) for k in range(shnum)]
    symtab = [sh for sh in secs if sh[1] == 2][0]          # SHT_SYMTAB
    strtab = secs[symtab[6]]
    sym = (ATTN_SYMBOL % head_dim).encode()
    parts = {}
    for k in range(symtab[5] // 24):
        st_name, _, _, st_shndx, st_value, st_size = struct.unpack_from("<IBBHQQ", elf, symtab[4] + 24 * k)
        a = strtab[4] + st_name
        name = elf[a: elf.index(b"\0", a)]
        if name in (sym, sym + b".kd"):
            sh = secs[st_shndx]
            fo = sh[4] + (st_value - sh[3])
            parts[name] = bytearray(elf[fo: fo + st_size])
    if len(parts) != 2:
        raise RuntimeError("attention kernel symbol not found in " + lib_path)
    kd = parts[sym + b".kd"]
    kd[16:24] = bytes(8)                                    # kernel_code_entry_byte_offset
    return hashlib.sha256(bytes(parts[sym]) + bytes(kd)).hexdigest()[:16]


if __name__ == "__main__":
    main()
