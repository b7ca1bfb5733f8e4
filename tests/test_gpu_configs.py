"""GPU parity at the full sizes of the four larger workloads (the mid layer
T=4096/d=2048/E=64/k=6/F=1024, the 384-expert V4-Flash-like layer
T=8192/d=4096/F=2048, its skewed multimodal variant and the hash-routed
T=32768 layer), in the launch configuration the benchmark times (packed
weights, one moe_forward call):

  - routing ids and weights bit-exact for every token, given the GPU's fp32
    router logits (the oracle consumes the exported logits);
  - the dispatch permutation (counts, offsets, dest, src) bit-exact and every
    gathered row byte-equal to its token row;
  - router logits on sampled rows within the fp32 accumulation bound;
  - the layer output (fp32 mode) within 1e-2 x RMS of the oracle: every
    token of the 64-expert layer; at the larger ones a token set that covers
    every non-empty expert and, for every m-tile of the expert GEMMs, its
    first and last row and the rows on both sides of each 32-row block
    boundary (plus the shared expert's tile boundaries and a seeded random
    sample);
    the bf16 output within one bf16 rounding of that bound.
Near-ties (k-th vs (k+1)-th biased score gap below 1e-6) are counted and
printed (they are bit-exact here because both sides use the same logits).
Route flips are counted and printed too: the tokens whose expert set under
the oracle's own fp64-accumulated logits differs from the set under the
GPU's fp32-accumulated logits.  A flip may only happen at a near-tie: the
k-th vs (k+1)-th biased-score gap of a flipped token must be within what the
logit difference can move two scores (sigmoid slope <= 1/4, so at most
0.5 x max |logit difference| of the row, plus a few score ulps).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (bits, host, bf16_f64, check_logits, check_rms, near_ties, route_flips,
                      free_cuda)
from sparse_moe_layer_04_amd import ops, workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def _opt(inp, key):
    return None if inp[key] is None else host(inp[key])


FM = 128   # activation rows per expert-GEMM tile


def flat_tile_split(n):
    """Rows per m-tile of an expert with n rows in the expert GEMM (every
    weight mode): the rows split evenly over ceil(n / 128) tiles, rounded up
    to 32."""
    mt = -(-n // FM)
    return (-(-n // mt) + 31) & ~31


_bf16_tile_split = _mx_tile_split = flat_tile_split


def tile_edge_rows(lo, hi, per):
    """Rows of the expert segment [lo, hi) at the edges of its m-tiles of
    `per` rows: each tile's first and last row and the rows on both sides of
    every 32-row block boundary inside it (each block is one MFMA column
    block of every wave)."""
    out = []
    for r0 in range(lo, hi, per):
        valid = min(per, hi - r0)
        out += [r0, r0 + valid - 1]
        for b in range(32, valid, 32):
            out += [r0 + b - 1, r0 + b]
    return out


def coverage_tokens(counts, offsets, src, split, T, rng, n_random=32):
    """Tokens whose outputs cover every non-empty expert and every m-tile
    edge of the routed expert GEMMs (rows of the dispatch order mapped to
    their tokens through src), the shared expert's tile edges (its single
    group of T rows) and n_random seeded random tokens."""
    rows = []
    for e in np.nonzero(counts)[0]:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows += tile_edge_rows(lo, hi, split(hi - lo))
    toks = [src[np.asarray(rows, np.int64)], np.asarray(tile_edge_rows(0, T, FM), np.int64),
            rng.choice(T, size=min(n_random, T), replace=False)]
    return np.unique(np.concatenate(toks).astype(np.int64))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_size(cfg):
    w = wl.WORKLOADS[cfg]
    print(f"\n[{w.name}] generating inputs", flush=True)
    inp = wl.make_inputs(w, DEV)
    layer = ops.MoeLayer.from_workload(w, inp, out_dtype=ops.OUT_F32, packed=True)
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device=DEV)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=DEV)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
    y = layer.forward(inp["x"], input_ids=inp["input_ids"], modality=inp["modality"],
                      logits=logits, ids=ids, w=wts)
    layer.cfg.out_dtype = ops.OUT_BF16
    y16 = layer.forward(inp["x"], input_ids=inp["input_ids"], modality=inp["modality"])
    torch.cuda.synchronize()
    assert int(layer.flags.item()) == 0

    lg = host(logits)
    bias, mod = _opt(inp, "score_bias"), _opt(inp, "modality")
    ids_in, tab = _opt(inp, "input_ids"), _opt(inp, "tid2eid")
    # routing: bit-exact on every token
    rid, rw, rf = oracle.route(lg, w.k, w.scale, bias=bias, modality=mod, input_ids=ids_in,
                               tid2eid=tab, mode=w.mode)
    assert rf == 0
    assert np.array_equal(host(ids), rid)
    assert np.array_equal(host(wts).view(np.uint32), rw.view(np.uint32))
    if w.mode == wl.MODE_TOPK:
        rows = bias[mod.astype(np.int64)] if (bias is not None and mod is not None and
                                             bias.shape[0] > 1) else bias
        print(f"[{w.name}] near-tie tokens (gap < 1e-6): {near_ties(lg, rows, w.k)}", flush=True)
        flips = route_flips(bits(inp["x"]), bits(inp["w_g"]), _opt(inp, "logit_offset"), lg,
                            bias, mod, rid, w.k)
        print(f"[{w.name}] route flips vs fp64 logits: {len(flips)} tokens"
              + "".join(f"; t={t} gap={g:.2e} (bound {b:.2e})" for t, g, b in flips[:8]),
              flush=True)
        assert all(g <= b for _, g, b in flips)

    # permutation: bit-exact, gathered rows byte-equal
    perm = ops.permute(ids, inp["x"], w.E)
    counts, offsets, dest, src, _ = oracle.permute(rid, w.E)
    assert np.array_equal(host(perm["counts"]), counts)
    assert np.array_equal(host(perm["offsets"]), offsets)
    assert np.array_equal(host(perm["dest"]), dest)
    assert np.array_equal(host(perm["src"]), src)
    xb = bits(inp["x"])
    assert np.array_equal(bits(perm["x_perm"]), xb[src])
    print(f"[{w.name}] expert rows: min {counts.min()} max {counts.max()} "
          f"empty {(counts == 0).sum()}", flush=True)
    del perm

    # router logits on sampled rows
    rng = np.random.default_rng(1000 + cfg)
    rows = np.sort(rng.choice(w.T, size=48, replace=False))
    check_logits(xb, bits(inp["w_g"]), _opt(inp, "logit_offset"), lg, rows)

    # layer output: every token of the 64-expert layer; at the larger ones
    # every non-empty expert and every m-tile edge of the expert GEMMs
    if cfg == 1:
        toks = np.arange(w.T, dtype=np.int64)
    else:
        toks = coverage_tokens(counts, offsets, src, _bf16_tile_split, w.T, rng)
    covered = np.unique(rid[toks])
    assert set(np.nonzero(counts)[0]) <= set(covered.tolist())
    shared = [bits(inp[k]) if inp[k] is not None else None for k in ("s_gate", "s_up", "s_down")]
    yref = oracle.tokens_forward(xb, toks, rid, rw, bits(inp["w_gate"]), bits(inp["w_up"]),
                                 bits(inp["w_down"]), *shared, w.clamp_limit, w.clamp_mode)
    rel = check_rms(host(y)[toks], yref)
    rms = np.sqrt(np.mean(yref ** 2))
    err16 = np.abs(bf16_f64(bits(y16))[toks] - yref)
    assert np.all(err16 <= 2.0 ** -8 * np.abs(yref) + 1e-2 * rms)
    print(f"[{w.name}, bf16 weights] {len(toks)} of {w.T} tokens, {len(covered)} experts "
          f"(all non-empty): max|y - y_oracle| / rms = {rel:.2e}", flush=True)
    del layer, inp, y, y16, logits, ids, wts
    free_cuda()


def _dequant_experts(m, experts, quant, dequant):
    """The oracle's dequantisation of the listed experts' matrices, in place
    (host threads over experts; each call is one C routine)."""
    import concurrent.futures as cf

    def one(e):
        q, ex = quant(m[e])
        m[e] = dequant(q, ex)

    with cf.ThreadPoolExecutor(max_workers=16) as ex:
        list(ex.map(one, [int(e) for e in experts]))


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_size_mx(cfg, fmt):
    """The MXFP8 and MXFP4 routed-weight modes at full size (the 64-expert
    layer, whose ~384-row experts split into two ~192-row tiles; the
    384-expert layer; the skewed multimodal one; and the hash-routed T=32768
    layer, whose experts take 64-wide stages), in the benchmark's launch
    configuration (--weights fp8 / fp4): routes bit-exact, and the outputs of
    a token set covering every non-empty expert and every m-tile edge (tiles
    split evenly in these modes) within 1e-2 x RMS of the oracle run on the
    oracle's own dequantisation of every expert's weights."""
    quant, dequant = ((oracle.quant_mxfp8, oracle.dequant_mxfp8) if fmt == "fp8" else
                      (oracle.quant_mxfp4, oracle.dequant_mxfp4))
    w = wl.WORKLOADS[cfg]
    print(f"\n[{w.name}, {fmt} weights] generating inputs", flush=True)
    inp = wl.make_inputs(w, DEV)
    layer = ops.MoeLayer.from_workload(w, inp, out_dtype=ops.OUT_F32, packed=fmt)
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device=DEV)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=DEV)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
    y = layer.forward(inp["x"], input_ids=inp["input_ids"], modality=inp["modality"],
                      logits=logits, ids=ids, w=wts)
    torch.cuda.synchronize()
    assert int(layer.flags.item()) == 0
    rid, rw, _ = oracle.route(host(logits), w.k, w.scale, bias=_opt(inp, "score_bias"),
                              modality=_opt(inp, "modality"), input_ids=_opt(inp, "input_ids"),
                              tid2eid=_opt(inp, "tid2eid"), mode=w.mode)
    assert np.array_equal(host(ids), rid)
    assert np.array_equal(host(wts).view(np.uint32), rw.view(np.uint32))
    counts, offsets, _, src, _ = oracle.permute(rid, w.E)
    rng = np.random.default_rng(77)
    toks = coverage_tokens(counts, offsets, src, _mx_tile_split, w.T, rng)
    experts = np.unique(rid[toks])
    assert set(np.nonzero(counts)[0]) <= set(experts.tolist())
    mats = {}
    for key in ("w_gate", "w_up", "w_down"):
        m = bits(inp[key])
        _dequant_experts(m, experts, quant, dequant)
        mats[key] = m
    shared = [bits(inp[k]) for k in ("s_gate", "s_up", "s_down")]
    yref = oracle.tokens_forward(bits(inp["x"]), toks, rid, rw, mats["w_gate"], mats["w_up"],
                                 mats["w_down"], *shared, w.clamp_limit, w.clamp_mode)
    rel = check_rms(host(y)[toks], yref)
    print(f"[{w.name}, {fmt} weights] {len(toks)} of {w.T} tokens, {len(experts)} experts "
          f"(all non-empty): max|y - y_oracle| / rms = {rel:.2e}", flush=True)
    del layer, inp, y, logits, ids, wts, mats
    free_cuda()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_size_a8w4(cfg):
    """The A8W4 mode (MXFP4 routed weights, MXFP8 activations on the scaled
    MX matrix cores; --weights a8w4) at full size: routes bit-exact, and the
    outputs of a token set covering every non-empty expert and every m-tile
    edge within tolerance of the oracle's A8W4 layer on its own
    quantisation of x, h and every covered expert's weights (tolerance as in
    test_gpu_a8w4: 5e-2 x RMS elementwise, 5e-3 relative Frobenius)."""
    w = wl.WORKLOADS[cfg]
    print(f"\n[{w.name}, a8w4] generating inputs", flush=True)
    inp = wl.make_inputs(w, DEV)
    layer = ops.MoeLayer.from_workload(w, inp, out_dtype=ops.OUT_F32, packed="a8w4")
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device=DEV)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=DEV)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
    y = layer.forward(inp["x"], input_ids=inp["input_ids"], modality=inp["modality"],
                      logits=logits, ids=ids, w=wts)
    torch.cuda.synchronize()
    assert int(layer.flags.item()) == 0
    rid, rw, _ = oracle.route(host(logits), w.k, w.scale, bias=_opt(inp, "score_bias"),
                              modality=_opt(inp, "modality"), input_ids=_opt(inp, "input_ids"),
                              tid2eid=_opt(inp, "tid2eid"), mode=w.mode)
    assert np.array_equal(host(ids), rid)
    assert np.array_equal(host(wts).view(np.uint32), rw.view(np.uint32))
    counts, offsets, _, src, _ = oracle.permute(rid, w.E)
    rng = np.random.default_rng(78)
    toks = coverage_tokens(counts, offsets, src, flat_tile_split, w.T, rng)
    experts = np.unique(rid[toks])
    assert set(np.nonzero(counts)[0]) <= set(experts.tolist())
    mats = {}
    for key in ("w_gate", "w_up", "w_down"):
        m = bits(inp[key])
        _dequant_experts(m, experts, oracle.quant_mxfp4, oracle.dequant_mxfp4)
        mats[key] = m
    shared = [bits(inp[k]) for k in ("s_gate", "s_up", "s_down")]
    yref = oracle.tokens_forward_a8w4(bits(inp["x"]), toks, rid, rw, mats["w_gate"],
                                      mats["w_up"], mats["w_down"], *shared, w.clamp_limit,
                                      w.clamp_mode)
    got = host(y)[toks].astype(np.float64)
    rel = check_rms(got, yref, tol=5e-2)
    fro = float(np.linalg.norm(got - yref) / np.linalg.norm(yref))
    assert fro <= 5e-3, fro
    print(f"[{w.name}, a8w4] {len(toks)} of {w.T} tokens, {len(experts)} experts "
          f"(all non-empty): max|y - y_oracle| / rms = {rel:.2e}, rel. Frobenius {fro:.2e}",
          flush=True)
    del layer, inp, y, logits, ids, wts, mats
    free_cuda()
