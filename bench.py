"""Benchmark of the MoE layer forward on one MI355X.

One step = one moe_forward call (router projection, routing, dispatch
permutation, routed + shared expert FFNs, combine) over the resident
synthetic batch of the chosen workload (default: the 384-expert top-6
V4-Flash-like layer, T=8192, d=4096, F=2048).  Prints one JSON line.

The K timed steps replay one captured forward (a HIP graph of the library's
kernels; --eager times K eager calls instead).  Per-stage times come from
HIP events recorded by the library around its stages on the launch stream
(moe_forward_timed) during K eager steps; the roofline object is for the
dominant kernel (longest stage).  The CPU baseline
times the C oracle on a bounded token sample on the host cores.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # FLOP/s, MI355X dense bf16 MFMA
PEAK_FP8 = 5.0e15          # FLOP/s, MI355X dense fp8 MFMA


def stage_work(w, n_nonempty, out_bytes=2, wbytes=2, abytes=2):
    """Algorithmic (minimum) HBM bytes and FLOPs per stage (wbytes: bytes per
    routed expert weight; MX weights also read one scale byte per 32; abytes:
    bytes per routed-GEMM activation, 1 for MXFP8 activations plus one scale
    byte per 32, whose quantisation of x is part of the permute stage)."""
    T, d, E, k, F, Fs = w.T, w.d, w.E, w.k, w.F, w.Fs
    N = T * k
    hash_mode = w.mode == 1
    st = {}
    st["router_gemm"] = (T * d * 2 + E * d * 2 + T * E * 4, 2.0 * T * d * E)
    # TopK reads every logit; Hash reads the token id, its table row and the
    # k logits at the table's ids; both write ids and weights
    route_bytes = (T * 4 + T * k * 4 + T * k * 4 if hash_mode else T * E * 4) + T * k * 8
    st["route"] = (route_bytes, 0.0)
    # the forward's permutation writes dest/src only (the routed gate/up GEMM
    # gathers the token rows through src)
    a_sc = 1.0 / 32 if abytes < 2 else 0.0
    st["permute"] = (N * 4 + 2 * N * 4 + (T * d * (2 + 1 + a_sc) if abytes < 2 else 0), 0.0)
    # routed gate/up: weights of the non-empty experts once, every routed row
    # of x once (gathered), h written once
    st["gate_up_routed"] = (n_nonempty * 2 * F * (d * wbytes + (d // 32 if wbytes < 2 else 0)) +
                            N * d * (abytes + a_sc) + N * F * (abytes + a_sc),
                            2.0 * N * d * 2 * F)
    st["gate_up_shared"] = (2 * Fs * d * 2 + T * d * 2 + T * Fs * 2, 2.0 * T * d * 2 * Fs)
    st["down_routed"] = (n_nonempty * d * (F * wbytes + (F // 32 if wbytes < 2 else 0)) +
                         N * F * (abytes + a_sc) + N * d * 4, 2.0 * N * F * d)
    st["down_shared"] = (d * Fs * 2 + T * Fs * 2 + T * d * 4, 2.0 * T * Fs * d)
    st["combine"] = (N * d * 4 + (T * d * 4 if Fs else 0) + N * 8 + T * d * out_bytes, 0.0)
    return st


# source files that define each stage's kernels: a recorded counter value
# stays valid only while these are unchanged
STAGE_SOURCES = {
    "router_gemm": ("router.hip", "moe_internal.h"),
    "route": ("route.hip", "moe_internal.h"),
    "permute": ("permute.hip", "moe_internal.h"),
    "gate_up_routed": ("gemm_flat.hip", "moe_internal.h"),
    "gate_up_shared": ("gemm_flat.hip", "moe_internal.h"),
    "down_routed": ("gemm_flat.hip", "moe_internal.h"),
    "down_shared": ("gemm_flat.hip", "moe_internal.h"),
    "combine": ("combine.hip", "moe_internal.h"),
}


def kernel_source_digest(stage):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_layer_04_amd", "csrc")
    for name in STAGE_SOURCES[stage]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(stage, workload_name):
    """Counter-derived HBM traffic of a stage's kernels per launch, if it was
    recorded (profiles/traffic.json) for the current sources of those
    kernels, else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get("kernels", {}).get(f"{workload_name}:{stage}")
    if not ent or ent.get("source_digest") != kernel_source_digest(stage):
        return None
    return ent.get("bytes_per_launch")


def routing_diagnostics(w, inp, logits, ids, gap=1e-6):
    """Near-ties and route flips of the benchmarked forward (TopK routing),
    computed after the timed region with plain torch fp64 arithmetic:
      near_ties   - tokens whose k-th and (k+1)-th biased scores, from the
                    forward's own fp32 logits, differ by less than `gap`;
      route_flips - tokens whose expert set under logits accumulated in fp64
                    (x W_g^T + offset) differs from the forward's set.
    None for hash routing (no ranking)."""
    import torch
    if w.mode == 1:
        return None
    bias = inp["score_bias"]
    rows = None
    if bias is not None:
        rows = bias.double()[inp["modality"].long()] if (
            inp["modality"] is not None and bias.shape[0] > 1) else bias.double()[:1]

    def ranked(lg):
        r = torch.sigmoid(lg.double())
        if rows is not None:
            r = r + rows
        return r

    r = ranked(logits)
    top = torch.topk(r, w.k + 1, dim=1).values
    near = int((top[:, w.k - 1] - top[:, w.k] < gap).sum().item())
    lg64 = inp["x"].double() @ inp["w_g"].double().T
    if inp["logit_offset"] is not None:
        lg64 = lg64 + inp["logit_offset"].double()
    ids64 = torch.topk(ranked(lg64), w.k, dim=1).indices
    flips = int((torch.sort(ids64, dim=1).values !=
                 torch.sort(ids.long(), dim=1).values).any(dim=1).sum().item())
    return {"near_ties": near, "route_flips": flips, "gap": gap,
            "how": "near_ties: k-th minus (k+1)-th biased score < gap under the forward's fp32 "
                   "logits; route_flips: tokens whose expert set under fp64-accumulated logits "
                   "differs from the forward's (torch fp64, outside the timed region)"}


def cpu_baseline(w, inp, budget_s, seed=123):
    """Time the oracle (gate logits -> route -> per-token layer output) on a
    token sample sized to take about `budget_s` seconds of host CPU."""
    import oracle
    from sparse_moe_layer_04_amd.workloads import bf16_bits
    host = lambda t: None if t is None else t.detach().cpu().numpy()
    x = bf16_bits(inp["x"])
    wg = bf16_bits(inp["w_g"])
    wgate, wup, wdown = (bf16_bits(inp[k]) for k in ("w_gate", "w_up", "w_down"))
    sh = [bf16_bits(inp[k]) if inp[k] is not None else None for k in ("s_gate", "s_up", "s_down")]
    off, bias, mod = host(inp["logit_offset"]), host(inp["score_bias"]), host(inp["modality"])
    ids_in, tab = host(inp["input_ids"]), host(inp["tid2eid"])
    rng = np.random.default_rng(seed)

    def run(n):
        tok = np.sort(rng.choice(w.T, size=n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        lg = oracle.gate_logits(x[tok], wg, off)
        ids, wts, _ = oracle.route(lg, w.k, w.scale, bias=bias,
                                   modality=None if mod is None else mod[tok],
                                   input_ids=None if ids_in is None else ids_in[tok],
                                   tid2eid=tab, mode=w.mode)
        full_ids = np.zeros((w.T, w.k), np.int32)
        full_w = np.zeros((w.T, w.k), np.float32)
        full_ids[tok], full_w[tok] = ids, wts
        oracle.tokens_forward(x, tok, full_ids, full_w, wgate, wup, wdown, *sh, w.clamp_limit,
                              w.clamp_mode)
        return time.perf_counter() - t0

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    probe_n = max(1, min(w.T, threads))
    t_probe = run(probe_n)
    n = int(max(probe_n, min(w.T, probe_n * budget_s / max(t_probe, 1e-6))))
    n = max(threads, (n // threads) * threads) if n >= threads else n
    n = min(n, w.T)
    t = run(n)
    return {"value": n / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {w.T} tokens (seeded sample): fp64 router projection, routing, "
                      f"and every routed + shared expert FFN of each sampled token; {t:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload index (0-4)")
    ap.add_argument("--out-dtype", choices=["bf16", "f32"], default="bf16")
    ap.add_argument("--layout", choices=["packed", "plain"], default="packed",
                    help="weight layout: packed once at load time (moe_pack_weights) or "
                         "the plain [out, in] matrices")
    ap.add_argument("--weights", choices=["bf16", "fp8", "fp4", "a8w4"], default="bf16",
                    help="routed expert weights: bf16, MXFP8 (E4M3 codes) or MXFP4 (E2M1 codes), "
                         "one power-of-two scale per 32 values of K (moe_pack_weights_fp8 / "
                         "_fp4; packed layout only); a8w4: MXFP4 weights and MXFP8 "
                         "activations on the scaled MX matrix cores")
    ap.add_argument("--eager", action="store_true",
                    help="time K eager moe_forward calls instead of K replays of one captured "
                         "forward (HIP graph); the per-stage breakdown comes from eager calls "
                         "either way")
    ap.add_argument("--extras", choices=["all", "none", "backward"], default="all",
                    help="after the forward's timing, also time the backward pieces, the weight "
                         "gradient and the whole layer backward (all), only the layer backward "
                         "(backward), or nothing (none: a fixed set of forward calls for "
                         "profiling)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle CPU work for the baseline (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU only (no expert-parallel path); --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    from sparse_moe_layer_04_amd import ops, workloads as wl

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    w = wl.WORKLOADS[args.config]
    print(f"# generating workload {w.name}", file=sys.stderr, flush=True)
    inp = wl.make_inputs(w, dev)
    out_dtype = ops.OUT_F32 if args.out_dtype == "f32" else ops.OUT_BF16
    if args.weights != "bf16" and args.layout != "packed":
        ap.error("--weights fp8 / fp4 needs --layout packed")
    layer = ops.MoeLayer.from_workload(w, inp, out_dtype=out_dtype,
                                       packed=args.weights if args.weights != "bf16" else
                                       args.layout == "packed")
    y = torch.empty((w.T, w.d), dtype=torch.float32 if out_dtype == ops.OUT_F32 else torch.bfloat16,
                    device=dev)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    fwd = lambda events=None: layer.forward(inp["x"], input_ids=inp["input_ids"],
                                            modality=inp["modality"], y=y, ids=ids, events=events)
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()

    nst = ops.FORWARD_STAGES
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)]
              for _ in range(args.steps)]
    for evs in events:             # materialise the event handles
        for e in evs:
            e.record()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        fwd(events[i])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    stage_ms = np.zeros(nst)
    for evs in events:
        for s in range(nst):
            stage_ms[s] += evs[s].elapsed_time(evs[s + 1])
    stage_ms /= args.steps
    assert int(layer.flags.item()) == 0, "device flagged invalid ids"

    ms_eager = ms
    if not args.eager:
        # one captured forward, replayed K times between the same barriers
        # (the first call's one-time kernel set-up ran in the warm-up)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fwd()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            graph.replay()
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / args.steps
        assert int(layer.flags.item()) == 0, "device flagged invalid ids"

    # The same forward with the 256 MB MALL overwritten before every call (a
    # 512 MiB fill between calls, outside the timed event pair), reported
    # beside the back-to-back figure: the gap is what cross-call cache reuse
    # is worth.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    n_cold = min(args.steps, 5)
    cold = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n_cold)]
    for i, (e0, e1) in enumerate(cold):
        flush.fill_(i + 1)
        e0.record()
        fwd()
        e1.record()
    torch.cuda.synchronize()
    ms_cold = sum(e0.elapsed_time(e1) for e0, e1 in cold) / n_cold
    del flush

    route_backward = combine_backward = swiglu_backward = down_dgrad = wgrad_down = None
    routing = None
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.extras == "all":
        # The routing backward (moe_route_backward: the routing weights' gradient
        # taken back to the logits) on this workload's own forward routes, timed
        # outside the forward step: 20 calls captured in one graph, replayed
        # between two events (each call is a few microseconds of device work,
        # less than the host cost of one call).
        lg_b = torch.empty((w.T, w.E), dtype=torch.float32, device=dev)
        ids_b = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
        wts_b = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
        layer.forward(inp["x"], input_ids=inp["input_ids"], modality=inp["modality"], logits=lg_b,
                      ids=ids_b, w=wts_b)
        dw_b = torch.randn((w.T, w.k), generator=gen, device=dev)
        dl_b = torch.empty((w.T, w.E), dtype=torch.float32, device=dev)
        ops.route_backward(lg_b, ids_b, dw_b, w.scale, out=dl_b)
        torch.cuda.synchronize()
        n_rb = 20
        rb_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(rb_graph):
            for _ in range(n_rb):
                ops.route_backward(lg_b, ids_b, dw_b, w.scale, out=dl_b)
        rb_graph.replay()
        torch.cuda.synchronize()
        e0.record()
        rb_graph.replay()
        e1.record()
        torch.cuda.synchronize()
        rb_ms = e0.elapsed_time(e1) / n_rb
        # ids, dw and the k gathered logits read; the whole d_logits row written
        rb_bytes = w.T * w.k * 12 + w.T * w.E * 4
        route_backward = {"ms": rb_ms, "GB/s": rb_bytes / rb_ms / 1e6,
                          "frac_of_hbm_peak": rb_bytes / rb_ms / 1e6 / (PEAK_HBM / 1e9),
                          "algorithmic_bytes": rb_bytes}
        # near-ties and route flips of this forward's routing (not timed)
        routing = routing_diagnostics(w, inp, lg_b, ids_b)
        del rb_graph, dl_b, lg_b

        # The combine backward (moe_combine_backward: the output gradient taken
        # to the expert outputs and the routing weights) at this workload's
        # shapes: the forward's routes and weights, random fp32 expert outputs
        # and output gradient; 5 calls between two events.
        # (dest of the forward's dispatch: each pair's row in the stable
        # expert-major order; setup data, computed here with torch)
        order = torch.argsort(ids_b.flatten().long(), stable=True)
        dest_b = torch.empty(w.T * w.k, dtype=torch.int32, device=dev)
        dest_b[order] = torch.arange(w.T * w.k, dtype=torch.int32, device=dev)
        del order
        yp_b = torch.randn((w.T * w.k, w.d), generator=gen, device=dev)
        dy_b = torch.randn((w.T, w.d), generator=gen, device=dev)
        dyp_b = torch.empty_like(yp_b)
        dwt_b = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
        ops.combine_backward(dy_b, yp_b, dest_b, wts_b, dy_perm=dyp_b, d_topk_w=dwt_b)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            ops.combine_backward(dy_b, yp_b, dest_b, wts_b, dy_perm=dyp_b, d_topk_w=dwt_b)
        e1.record()
        torch.cuda.synchronize()
        cb_ms = e0.elapsed_time(e1) / 5
        # dy and every routed expert output read, every expert-output gradient
        # written, dest / w read and d_topk_w written
        cb_bytes = w.T * w.d * 4 + 2 * w.T * w.k * w.d * 4 + w.T * w.k * 12
        combine_backward = {"ms": cb_ms, "GB/s": cb_bytes / cb_ms / 1e6,
                            "frac_of_hbm_peak": cb_bytes / cb_ms / 1e6 / (PEAK_HBM / 1e9),
                            "algorithmic_bytes": cb_bytes}
        del yp_b, dy_b, dyp_b, dest_b

        # The clamped-SwiGLU backward (moe_swiglu_backward) at this workload's
        # [T k, F] pre-activation shape: random fp32 gate/up pre-activations and
        # h gradient; 5 calls between two events.
        sb_shape = (w.T * w.k, w.F)
        g_sb = torch.randn(sb_shape, generator=gen, device=dev) * 4
        u_sb = torch.randn(sb_shape, generator=gen, device=dev) * 4
        dh_sb = torch.randn(sb_shape, generator=gen, device=dev)
        dg_sb, du_sb = torch.empty_like(g_sb), torch.empty_like(g_sb)
        ops.swiglu_backward(g_sb, u_sb, dh_sb, w.clamp_limit, w.clamp_mode, dgate=dg_sb, dup=du_sb)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            ops.swiglu_backward(g_sb, u_sb, dh_sb, w.clamp_limit, w.clamp_mode, dgate=dg_sb,
                                dup=du_sb)
        e1.record()
        torch.cuda.synchronize()
        sb_ms = e0.elapsed_time(e1) / 5
        sb_bytes = 20 * w.T * w.k * w.F          # three fp32 inputs read, two written
        swiglu_backward = {"ms": sb_ms, "GB/s": sb_bytes / sb_ms / 1e6,
                           "frac_of_hbm_peak": sb_bytes / sb_ms / 1e6 / (PEAK_HBM / 1e9),
                           "algorithmic_bytes": sb_bytes}
        del g_sb, u_sb, dh_sb, dg_sb, du_sb

        # The down projection's input gradient dH = dY W_down per expert
        # (moe_grouped_gemm_packed with W_down^T packed once) at this workload's
        # group sizes: random bf16 dY; 3 calls between two events.
        counts_b = torch.bincount(ids_b.flatten().long(), minlength=w.E)
        offs_b = torch.zeros(w.E + 1, dtype=torch.int32, device=dev)
        offs_b[1:] = torch.cumsum(counts_b, 0).to(torch.int32)
        wdT_b = ops.pack_weights(inp["w_down"].transpose(1, 2).contiguous(), 256)
        dY_b = torch.randn((w.T * w.k, w.d), generator=gen, device=dev).to(torch.bfloat16)
        dH_b = torch.empty((w.T * w.k, w.F), dtype=torch.float32, device=dev)
        ops.grouped_gemm_packed(dY_b, offs_b, wdT_b, w.E, w.F, out=dH_b)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(3):
            ops.grouped_gemm_packed(dY_b, offs_b, wdT_b, w.E, w.F, out=dH_b)
        e1.record()
        torch.cuda.synchronize()
        dg_ms = e0.elapsed_time(e1) / 3
        nz_b = int((counts_b > 0).sum().item())
        dg_flops = 2.0 * w.T * w.k * w.d * w.F
        dg_bytes = nz_b * w.F * w.d * 2 + w.T * w.k * w.d * 2 + w.T * w.k * w.F * 4
        down_dgrad = {"ms": dg_ms, "TFLOP/s": dg_flops / dg_ms / 1e9,
                      "GB/s": dg_bytes / dg_ms / 1e6,
                      "frac_of_hbm_peak": dg_bytes / dg_ms / 1e6 / (PEAK_HBM / 1e9),
                      "frac_of_mfma_peak": dg_flops / dg_ms / 1e9 / (PEAK_BF16 / 1e12),
                      "algorithmic_bytes": dg_bytes, "flops": dg_flops}
        del wdT_b, dH_b

        # The down projection's weight gradient dW_down[e] = dY_e^T H_e
        # (moe_grouped_wgrad) at this workload's group sizes: random bf16 dY and
        # H; 3 calls between two events.
        H_b = torch.randn((w.T * w.k, w.F), generator=gen, device=dev).to(torch.bfloat16)
        dW_b = torch.empty((w.E, w.d, w.F), dtype=torch.float32, device=dev)
        ops.grouped_wgrad(dY_b, H_b, offs_b, out=dW_b)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(3):
            ops.grouped_wgrad(dY_b, H_b, offs_b, out=dW_b)
        e1.record()
        torch.cuda.synchronize()
        wg_ms = e0.elapsed_time(e1) / 3
        wg_flops = 2.0 * w.T * w.k * w.d * w.F
        # every dW entry written once (fp32), dY and H read once
        wg_bytes = w.E * w.d * w.F * 4 + w.T * w.k * (w.d + w.F) * 2
        wgrad_down = {"ms": wg_ms, "TFLOP/s": wg_flops / wg_ms / 1e9,
                      "GB/s": wg_bytes / wg_ms / 1e6,
                      "frac_of_hbm_peak": wg_bytes / wg_ms / 1e6 / (PEAK_HBM / 1e9),
                      "frac_of_mfma_peak": wg_flops / wg_ms / 1e9 / (PEAK_BF16 / 1e12),
                      "algorithmic_bytes": wg_bytes, "flops": wg_flops}
        del dY_b, H_b, dW_b
        torch.cuda.empty_cache()

    # The whole layer backward (moe_backward: the forward's intermediates
    # recomputed, then every gradient) for a random fp32 output gradient;
    # 1 warm-up call (it also packs the transposed weights once), then 3
    # calls between two events.
    layer_backward = None
    if args.extras in ("all", "backward") and args.weights == "bf16" and args.layout == "packed":
        dyb = torch.randn((w.T, w.d), generator=gen, device=dev)
        grads = layer.backward(inp["x"], dyb, input_ids=inp["input_ids"],
                               modality=inp["modality"])
        torch.cuda.synchronize()
        e0.record()
        for _ in range(3):
            layer.backward(inp["x"], dyb, input_ids=inp["input_ids"], modality=inp["modality"],
                           grads=grads)
        e1.record()
        torch.cuda.synchronize()
        lb_ms = e0.elapsed_time(e1) / 3
        assert int(layer.flags.item()) == 0, "device flagged invalid ids"
        # forward recomputation (expert products once) plus the input- and
        # weight-gradient products: 3x the forward's FLOPs on the experts
        fw_flops = 2.0 * w.T * (w.k * 3 * w.d * w.F + 3 * w.d * w.Fs)
        layer_backward = {"ms": lb_ms, "tokens/s": w.T / (lb_ms * 1e-3),
                          "TFLOP/s": 3 * fw_flops / lb_ms / 1e9,
                          "note": "forward recomputed inside; 3x the expert FFN FLOPs"}
        del grads, dyb
        layer.bw = layer.bworkspace = None
        torch.cuda.empty_cache()

    counts = torch.bincount(ids.flatten().long(), minlength=w.E).cpu().numpy()
    n_nonempty = int((counts > 0).sum())
    work = stage_work(w, n_nonempty, 4 if out_dtype == ops.OUT_F32 else 2,
                      wbytes={"bf16": 2, "fp8": 1, "fp4": 0.5, "a8w4": 0.5}[args.weights],
                      abytes=1 if args.weights == "a8w4" else 2)
    # matrix-core peak of the routed GEMMs: bf16, or fp8 for MXFP8 activations
    peak_mm = PEAK_FP8 if args.weights == "a8w4" else PEAK_BF16
    stages = {}
    for s, name in enumerate(ops.STAGE_NAMES):
        b, f = work[name]
        t = stage_ms[s] * 1e-3
        routed = name in ("gate_up_routed", "down_routed")
        bound = "mfma" if f > 0 and f / b > (peak_mm if routed else PEAK_BF16) / PEAK_HBM else "hbm"
        stages[name] = {"ms": round(float(stage_ms[s]), 4), "GB/s": round(b / t / 1e9, 1) if t else None,
                        "TFLOP/s": round(f / t / 1e12, 1) if t and f else None, "bound": bound}
    dom = max(range(nst), key=lambda s: stage_ms[s])
    dname = ops.STAGE_NAMES[dom]
    b, f = work[dname]
    t = stage_ms[dom] * 1e-3
    if stages[dname]["bound"] == "mfma":
        pk = peak_mm if dname in ("gate_up_routed", "down_routed") else PEAK_BF16
        roof = {"bound": "mfma", "achieved": f / t / 1e12, "peak": pk / 1e12,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": b / t / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = load_traffic(dname, w.name) if args.weights == "bf16" else None
    roof["kernel"] = dname
    roof["algorithmic_bytes"] = b
    roof["flops"] = f
    roof["avg_launch_ms"] = float(stage_ms[dom])

    gg = ("gate_up_routed", "down_routed")
    gg_t = sum(stage_ms[ops.STAGE_NAMES.index(n)] for n in gg) * 1e-3
    gg_f = sum(work[n][1] for n in gg)

    res = {
        "metric": "MoE fwd tokens/s + grouped-GEMM TFLOP/s (% of bf16 MFMA peak), 1 MI355X",
        "value": w.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_cold_mall": ms_cold,
        "ms_per_step_eager": ms_eager,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "bf16 activations, MXFP8 (E4M3) routed weights",
                  "fp4": "bf16 activations, MXFP4 (E2M1) routed weights",
                  "a8w4": "MXFP8 (E4M3) activations x MXFP4 (E2M1) routed weights on the "
                          "scaled MX matrix cores; router and shared expert bf16"}[args.weights],
        "data": "synthetic",
        "config": dict(w.describe(), out_dtype=args.out_dtype, weight_layout=args.layout,
                       routed_weights=args.weights, graph=not args.eager,
                       non_empty_experts=n_nonempty,
                       max_rows_per_expert=int(counts.max())),
        "grouped_gemm_tflops": gg_f / gg_t / 1e12,
        "grouped_gemm_mfma_frac": gg_f / gg_t / peak_mm,
        "roofline": roof,
        "stages": stages,
        "route_backward": route_backward,
        "combine_backward": combine_backward,
        "swiglu_backward": swiglu_backward,
        "down_dgrad": down_dgrad,
        "wgrad_down": wgrad_down,
        "layer_backward": layer_backward,
        "routing": routing,
    }
    if args.cpu_budget > 0:
        print("# timing the CPU oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
