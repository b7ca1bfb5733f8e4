"""GPU parity of the MXFP8 and MXFP4 routed-expert weight modes (E4M3 / E2M1
codes, one power-of-two scale per 32 values of K; moe_pack_weights_fp8 /
_fp4 + moe_forward with packed = MOE_WEIGHTS_FP8 / _FP4) against the oracle:

  - quantisation: codes and block scales bit-exact against the oracle's MX
    quantiser, on random rows plus zero, huge, tiny, saturating and tie
    blocks, every code and scale at its place in the packed layout and
    padding rows zero;
  - forward: routes bit-exact and y within 1e-2 x RMS of the oracle run on
    the dequantised weights (exact bf16 values);
  - the fp8 forward is bit-equal to the bf16 packed forward on the
    dequantised weights (codes and scale decode exactly to those bf16
    values, and the MFMA chain is the same).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bits, host, bf16_f64, case_id, check_rms
from sparse_moe_layer_04_amd import ops, workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def unpack_codes(codes, G, N, K, P):
    """[G][ceil(N/P)][K/64][P/32][2][64][16] -> [G, ceil(N/P)*P, K] codes."""
    npan = (N + P - 1) // P
    a = codes.reshape(G, npan, K // 64, P // 32, 2, 2, 32, 2, 8)
    # axes: g, panel, s, b, c, lane_hi, lane_lo, h, i ->
    #       g, panel, b, lane_lo | s, c, h, lane_hi, i
    a = a.transpose(0, 1, 3, 6, 2, 4, 7, 5, 8)
    return a.reshape(G, npan * P, K)


def unpack_codes_fp4(codes, G, N, K, P):
    """[G][ceil(N/P)][K/32][P/32][64][8 B] two codes per byte (low nibble
    first) -> [G, ceil(N/P)*P, K] codes."""
    npan = (N + P - 1) // P
    a = codes.reshape(G, npan, K // 32, P // 32, 2, 32, 2, 4)
    # axes: g, panel, kb, b, lane_hi, lane_lo, word, byte (+ nibble)
    n = np.stack([a & 15, a >> 4], axis=-1).reshape(G, npan, K // 32, P // 32, 2, 32, 2, 8)
    # column of the block = 16 word + 8 lane_hi + nibble
    n = n.transpose(0, 1, 3, 5, 2, 6, 4, 7)
    return n.reshape(G, npan * P, K)


FORMATS = {
    "fp8": (lambda w, P: ops.pack_weights_fp8(w, P), unpack_codes, oracle.quant_mxfp8,
            oracle.dequant_mxfp8),
    "fp4": (lambda w, P: ops.pack_weights_fp4(w, P), unpack_codes_fp4, oracle.quant_mxfp4,
            oracle.dequant_mxfp4),
}


def unpack_scales(scales, G, N, K, P):
    """[G][ceil(N/P)][K/32][P/32][32] scale bytes -> block exponents X
    [G, ceil(N/P)*P, K/32]."""
    npan = (N + P - 1) // P
    a = scales.reshape(G, npan, K // 32, P // 32, 32).transpose(0, 1, 3, 4, 2)
    return a.reshape(G, npan * P, K // 32).astype(np.int32) - 127


def weights_with_special_rows(G, N, K, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((G, N, K)) / np.sqrt(K)).astype(np.float32)
    w[0, 0] = 0.0                                     # zero row
    w[0, 1] *= 2.0 ** 40                              # huge row
    w[0, 2] *= 2.0 ** -60                             # tiny row (subnormal codes)
    w[0, 3] *= 2.0 ** -115                            # exponent clamped at -110
    w[0, 4, :32] = 500.0                              # saturating block
    w[0, 4, 5] = 1.0
    # ties: consecutive E4M3 values and their midpoints, scaled by 2^-5,
    # with the row maximum exactly 448 * 2^-5
    vals = sorted({oracle.e4m3_decode(c) for c in range(0x7F)})
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    row = np.resize(np.array(vals + mids, np.float64), K) * 2.0 ** -5
    row[0] = 448.0 * 2.0 ** -5
    row[1::2] *= -1
    w[G - 1, N - 1] = row.astype(np.float32)
    b = (w.view(np.uint32) >> 16).astype(np.uint16)   # bf16 (truncation; exact for the ties)
    return b


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
@pytest.mark.parametrize("G,N,K,P", [(1, 64, 64, 128), (3, 200, 192, 128), (2, 256, 128, 256),
                                     (5, 96, 320, 256)])
def test_pack_weights_mx(G, N, K, P, fmt):
    pack, unpack, quant, _ = FORMATS[fmt]
    wb = weights_with_special_rows(G, N, K, seed=G * 1000 + N)
    w = torch.from_numpy(wb.view(np.int16)).to(DEV).view(torch.bfloat16)
    codes, scales = pack(w, P)
    torch.cuda.synchronize()
    q_ref, x_ref = quant(wb.reshape(G * N, K))
    got = unpack(host(codes), G, N, K, P)
    assert np.array_equal(got[:, :N].reshape(G * N, K), q_ref)
    assert not got[:, N:].any()
    xs = unpack_scales(host(scales), G, N, K, P)
    assert np.array_equal(xs[:, :N].reshape(G * N, K // 32), x_ref)


FP8_CASES = [
    wl.WORKLOADS[0],
    wl.small(T=300, d=256, E=16, k=4, F=192, seed=11, scale=2.5, F_shared=128),
    wl.small(T=515, d=128, E=64, k=6, F=64, seed=12, n_bias=2, vision_spans=2, span_len=100,
             zipf_expert_s=1.2),
    wl.small(T=400, d=192, E=32, k=6, F=128, seed=13, scale=2.5, mode=wl.MODE_HASH, V=500,
             zipf_token_s=1.1),
    wl.small(T=600, d=128, E=8, k=2, F=128, seed=15, scale=1.0),   # 2-3 m-tiles per expert
    wl.small(T=700, d=128, E=1024, k=8, F=64, seed=16, scale=2.5),  # E and k at their maxima
    wl.small(T=1, d=256, E=64, k=6, F=128, seed=19, scale=2.5),     # one token
    wl.small(T=300, d=256, E=16, k=4, F=192, seed=18, scale=2.5, clamp_limit=0.5,
             clamp_mode=1),                                          # the clamp saturates
]


def _dequantised(inp, fmt="fp8"):
    """inputs with the routed matrices replaced by their dequantised MX
    weights (exact bf16 values, from the oracle's quantiser)."""
    _, _, quant, dequant = FORMATS[fmt]
    out = dict(inp)
    for key in ("w_gate", "w_up", "w_down"):
        wb = bits(inp[key])
        q, x = quant(wb.reshape(-1, wb.shape[-1]))
        deq = dequant(q, x).reshape(wb.shape)
        out[key] = torch.from_numpy(deq.view(np.int16)).to(DEV).view(torch.bfloat16)
    return out


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
@pytest.mark.parametrize("w", FP8_CASES, ids=case_id)
def test_forward_mx(w, fmt):
    inp = wl.make_inputs(w, DEV)
    deq = _dequantised(inp, fmt)
    layer = ops.MoeLayer.from_workload(w, inp, out_dtype=ops.OUT_F32, packed=fmt)
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device=DEV)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=DEV)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
    y = layer.forward(inp["x"], input_ids=inp["input_ids"], modality=inp["modality"],
                      logits=logits, ids=ids, w=wts)
    # the bf16 packed forward on the dequantised weights: bit-equal
    ref_layer = ops.MoeLayer.from_workload(w, deq, out_dtype=ops.OUT_F32, packed=True)
    y_deq = ref_layer.forward(inp["x"], input_ids=inp["input_ids"], modality=inp["modality"])
    torch.cuda.synchronize()
    assert int(layer.flags.item()) == 0
    assert torch.equal(y.view(torch.int32), y_deq.view(torch.int32))
    # oracle on the dequantised weights, fed the GPU's logits
    opt = lambda key: None if inp[key] is None else host(inp[key])
    shared = [bits(inp[k]) if inp[k] is not None else None for k in ("s_gate", "s_up", "s_down")]
    ref = oracle.forward(bits(inp["x"]), host(logits), w.k, w.scale, bits(deq["w_gate"]),
                         bits(deq["w_up"]), bits(deq["w_down"]), *shared, w.clamp_limit,
                         w.clamp_mode, bias=opt("score_bias"), modality=opt("modality"),
                         input_ids=opt("input_ids"), tid2eid=opt("tid2eid"), mode=w.mode)
    assert np.array_equal(host(ids), ref["ids"])
    assert np.array_equal(host(wts).view(np.uint32), ref["w"].view(np.uint32))
    check_rms(host(y), ref["y"])


# expert row counts at every tile-shape boundary of the expert GEMM (empty,
# single rows, 16-row DMA groups, 128 / 192 / 256-row tiles and one row past
# each: both stage widths, multi-tile experts)
EXACT_COUNTS = [0, 1, 16, 17, 127, 128, 129, 191, 192, 193, 255, 256, 257, 384, 385, 512, 513,
                700]


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
@pytest.mark.parametrize("d,F,k", [(128, 64, 2), (256, 192, 4)])
def test_forward_mx_exact_group_sizes(d, F, k, fmt):
    slots = np.repeat(np.arange(len(EXACT_COUNTS), dtype=np.int32), EXACT_COUNTS)
    T = len(slots) // k
    table = np.ascontiguousarray(slots.reshape(k, T).T)
    w = wl.small(T=T, d=d, E=len(EXACT_COUNTS), k=k, F=F, seed=30 + k, scale=2.5,
                 mode=wl.MODE_HASH, V=T)
    inp = wl.make_inputs(w, DEV)
    inp["input_ids"] = torch.arange(T, dtype=torch.int32, device=DEV)
    inp["tid2eid"] = torch.from_numpy(table).to(DEV)
    deq = _dequantised(inp, fmt)
    layer = ops.MoeLayer.from_workload(w, inp, out_dtype=ops.OUT_F32, packed=fmt)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=DEV)
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device=DEV)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
    y = layer.forward(inp["x"], input_ids=inp["input_ids"], logits=logits, ids=ids, w=wts)
    ref_layer = ops.MoeLayer.from_workload(w, deq, out_dtype=ops.OUT_F32, packed=True)
    y_deq = ref_layer.forward(inp["x"], input_ids=inp["input_ids"])
    torch.cuda.synchronize()
    assert np.array_equal(np.bincount(host(ids).ravel(), minlength=w.E), EXACT_COUNTS)
    assert torch.equal(y.view(torch.int32), y_deq.view(torch.int32))
    shared = [bits(inp[k]) for k in ("s_gate", "s_up", "s_down")]
    ref = oracle.forward(bits(inp["x"]), host(logits), w.k, w.scale, bits(deq["w_gate"]),
                         bits(deq["w_up"]), bits(deq["w_down"]), *shared, w.clamp_limit,
                         w.clamp_mode, input_ids=host(inp["input_ids"]), tid2eid=table,
                         mode=w.mode)
    assert np.array_equal(host(ids), ref["ids"])
    check_rms(host(y), ref["y"])
