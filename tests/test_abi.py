"""The C-ABI library loads, exports every function include/moe.h declares, and
rejects bad arguments on the host before any launch (no GPU needed: every
case below returns before the first HIP call)."""
import ctypes

import pytest

from sparse_moe_layer_04_amd import ops

ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_ALIGN = -1, -2, -3, -4, -5, -6


@pytest.fixture(scope="module")
def L():
    return ops.lib()


def test_exports_every_declared_function(L):
    names = ops.declared_functions()
    assert {"moe_gate_logits", "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
            "moe_forward"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in (0, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_ALIGN):
        s = L.moe_status_string(code).decode()
        assert s and s != "unknown status"
    assert L.moe_status_string(-99).decode() == "unknown status"


FAKE = 0x10000  # an aligned non-NULL address; never dereferenced (checks fail first)


def route(L, T=4, E=8, k=2, n_bias=0, V=0, mode=0, scale=1.0, logits=FAKE, bias=None, ids=FAKE,
          w=FAKE, input_ids=None, tid2eid=None):
    return L.moe_route(logits, bias, None, input_ids, tid2eid, T, E, k, n_bias, V, mode,
                       ctypes.c_float(scale), ids, w, None, None)


def test_route_validation(L):
    assert route(L, k=0) == ERR_SHAPE
    assert route(L, E=0) == ERR_SHAPE
    assert route(L, T=-1) == ERR_SHAPE
    assert route(L, k=9, E=16) == ERR_UNSUPPORTED
    assert route(L, k=3, E=2) == ERR_UNSUPPORTED
    assert route(L, E=2000) == ERR_UNSUPPORTED
    assert route(L, mode=7) == ERR_UNSUPPORTED
    assert route(L, scale=float("nan")) == ERR_SHAPE
    assert route(L, logits=None) == ERR_NULL
    assert route(L, ids=None) == ERR_NULL
    assert route(L, n_bias=1, bias=None) == ERR_NULL
    assert route(L, n_bias=3, bias=FAKE) == ERR_SHAPE
    assert route(L, mode=1, input_ids=None, tid2eid=FAKE, V=10) == ERR_NULL
    assert route(L, mode=1, input_ids=FAKE, tid2eid=FAKE, V=0) == ERR_SHAPE
    assert route(L, T=0, logits=None, ids=None, w=None) == 0   # empty: nothing to do


def test_route_backward_validation(L):
    def rb(T=4, E=8, k=2, scale=1.0, logits=FAKE, ids=FAKE, dw=FAKE, out=FAKE):
        return L.moe_route_backward(logits, ids, dw, T, E, k, ctypes.c_float(scale), out, None,
                                    None)
    assert rb(k=0) == ERR_SHAPE
    assert rb(E=0) == ERR_SHAPE
    assert rb(T=-1) == ERR_SHAPE
    assert rb(k=9, E=16) == ERR_UNSUPPORTED
    assert rb(k=3, E=2) == ERR_UNSUPPORTED
    assert rb(E=2000) == ERR_UNSUPPORTED
    assert rb(scale=float("nan")) == ERR_SHAPE
    assert rb(logits=None) == ERR_NULL
    assert rb(ids=None) == ERR_NULL
    assert rb(dw=None) == ERR_NULL
    assert rb(out=None) == ERR_NULL
    assert rb(T=0, logits=None, ids=None, dw=None, out=None) == 0


def test_gate_logits_validation(L):
    assert L.moe_gate_logits(FAKE, FAKE, None, 4, 100, 8, FAKE, None) == ERR_UNSUPPORTED
    assert L.moe_gate_logits(FAKE, FAKE, None, 4, 32, 8, FAKE, None) == ERR_SHAPE
    assert L.moe_gate_logits(None, FAKE, None, 4, 128, 8, FAKE, None) == ERR_NULL
    assert L.moe_gate_logits(FAKE + 8, FAKE, None, 4, 128, 8, FAKE, None) == ERR_ALIGN
    assert L.moe_gate_logits(None, None, None, 0, 128, 8, None, None) == 0


def test_permute_validation(L):
    need = L.moe_permute_workspace_size(16, 2, 8)
    assert need > 0
    args = lambda **kw: [kw.get("ids", FAKE), kw.get("x", FAKE), kw.get("T", 16), kw.get("d", 64),
                         kw.get("E", 8), kw.get("k", 2), FAKE, FAKE, FAKE, FAKE,
                         kw.get("xp", FAKE), None, kw.get("ws", FAKE), kw.get("wsb", need), None]
    assert L.moe_permute(*args(ws=None)) == ERR_NULL
    assert L.moe_permute(*args(wsb=need - 1)) == ERR_WORKSPACE
    assert L.moe_permute(*args(ws=FAKE + 16)) == ERR_WORKSPACE
    assert L.moe_permute(*args(d=12)) == ERR_UNSUPPORTED
    assert L.moe_permute(*args(k=9)) == ERR_UNSUPPORTED
    assert L.moe_permute(*args(E=0)) == ERR_SHAPE
    assert L.moe_permute(*args(x=FAKE + 2)) == ERR_ALIGN
    assert L.moe_permute(*args(ids=None)) == ERR_NULL


@pytest.mark.parametrize("entry", ["moe_expert_ffn", "moe_expert_ffn_packed"])
def test_expert_ffn_validation(L, entry):
    def ffn(G=2, rows=10, d=128, F=64, L_=10.0, mode=0, a=FAKE, h=FAKE, off=FAKE):
        return getattr(L, entry)(a, off, G, rows, d, F, FAKE, FAKE, FAKE, ctypes.c_float(L_),
                                 mode, h, FAKE, None)
    assert ffn(G=0) == ERR_SHAPE
    assert ffn(G=5000) == ERR_UNSUPPORTED
    assert ffn(d=96) == ERR_UNSUPPORTED
    assert ffn(d=4194240 + 64) == ERR_UNSUPPORTED
    assert ffn(F=4194240 + 64) == ERR_UNSUPPORTED
    assert ffn(F=32) == ERR_SHAPE
    assert ffn(L_=0.0) == ERR_SHAPE
    assert ffn(L_=float("nan")) == ERR_SHAPE
    assert ffn(mode=2) == ERR_UNSUPPORTED
    assert ffn(a=None) == ERR_NULL
    assert ffn(off=None) == ERR_NULL
    assert ffn(h=FAKE + 4) == ERR_ALIGN
    assert ffn(rows=0, a=None) == 0


def test_pack_validation(L):
    assert L.moe_packed_weight_bytes(2, 40, 128, 128) == 2 * 128 * 128 * 2   # rows padded
    assert L.moe_packed_weight_bytes(2, 300, 64, 256) == 2 * 512 * 64 * 2
    assert L.moe_packed_weight_bytes(1, 8, 100, 128) == 0
    assert L.moe_packed_weight_bytes(1, 8, 128, 64) == 0
    assert L.moe_pack_weights(FAKE, 1, 8, 100, 128, FAKE, None) == ERR_UNSUPPORTED
    assert L.moe_pack_weights(FAKE, 1, 8, 128, 32, FAKE, None) == ERR_UNSUPPORTED
    assert L.moe_pack_weights(FAKE, 0, 8, 128, 128, FAKE, None) == ERR_SHAPE
    assert L.moe_pack_weights(None, 1, 8, 128, 128, FAKE, None) == ERR_NULL
    assert L.moe_pack_weights(FAKE, 1, 8, 128, 256, FAKE + 2, None) == ERR_ALIGN
    assert L.moe_packed_fp8_weight_bytes(2, 100, 128, 128) == 2 * 128 * 128
    assert L.moe_packed_fp8_weight_bytes(1, 8, 100, 128) == 0
    assert L.moe_packed_fp8_scale_bytes(2, 100, 128, 128) == 2 * 128 * 128 // 32
    assert L.moe_packed_fp4_weight_bytes(2, 100, 128, 128) == 2 * 128 * 128 // 2
    assert L.moe_pack_weights_fp4(FAKE, 1, 8, 100, 128, FAKE, FAKE, None) == ERR_UNSUPPORTED
    assert L.moe_pack_weights_fp4(FAKE, 1, 8, 128, 128, FAKE, None, None) == ERR_NULL
    assert L.moe_pack_weights_fp4(FAKE, 1, 8, 128, 256, FAKE + 2, FAKE, None) == ERR_ALIGN
    assert L.moe_pack_weights_fp8(FAKE, 1, 8, 100, 128, FAKE, FAKE, None) == ERR_UNSUPPORTED
    assert L.moe_pack_weights_fp8(FAKE, 0, 8, 128, 128, FAKE, FAKE, None) == ERR_SHAPE
    assert L.moe_pack_weights_fp8(FAKE, 1, 8, 128, 128, FAKE, None, None) == ERR_NULL
    assert L.moe_pack_weights_fp8(FAKE, 1, 8, 128, 256, FAKE + 2, FAKE, None) == ERR_ALIGN


def test_quantize_mxfp8_validation(L):
    assert L.moe_quantize_mxfp8(FAKE, 4, 48, FAKE, FAKE, None) == ERR_SHAPE      # K % 32
    assert L.moe_quantize_mxfp8(FAKE, -1, 64, FAKE, FAKE, None) == ERR_SHAPE
    assert L.moe_quantize_mxfp8(FAKE, 4, 0, FAKE, FAKE, None) == ERR_SHAPE
    assert L.moe_quantize_mxfp8(FAKE, 1 << 35, 64, FAKE, FAKE, None) == ERR_SHAPE
    assert L.moe_quantize_mxfp8(None, 4, 64, FAKE, FAKE, None) == ERR_NULL
    assert L.moe_quantize_mxfp8(FAKE, 4, 64, FAKE, None, None) == ERR_NULL
    assert L.moe_quantize_mxfp8(FAKE + 2, 4, 64, FAKE, FAKE, None) == ERR_ALIGN
    assert L.moe_quantize_mxfp8(FAKE, 4, 64, FAKE + 8, FAKE, None) == ERR_ALIGN
    assert L.moe_quantize_mxfp8(None, 0, 64, None, None, None) == 0            # nothing to do


def test_expert_ffn_a8w4_validation(L):
    def call(G=2, rows=8, d=128, F=128, a8=FAKE, y=FAKE, hs=FAKE):
        return L.moe_expert_ffn_a8w4(a8, FAKE, FAKE, G, rows, d, F, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, 10.0, 0, FAKE, hs, y, None)
    assert call(G=0) == ERR_SHAPE
    assert call(d=64) == ERR_UNSUPPORTED                # d and F multiples of 128
    assert call(F=192) == ERR_UNSUPPORTED
    assert call(G=1 << 20) == ERR_UNSUPPORTED
    assert call(a8=None) == ERR_NULL
    assert call(y=FAKE + 4) == ERR_ALIGN
    assert call(hs=FAKE + 2) == ERR_ALIGN
    assert call(rows=0, a8=None) == 0


def test_combine_validation(L):
    def comb(T=4, d=64, k=2, rows=8, out=0, yp=FAKE, y=FAKE):
        return L.moe_combine(yp, FAKE, FAKE, None, T, d, k, rows, out, y, None)
    assert comb(k=0) == ERR_SHAPE
    assert comb(k=9) == ERR_UNSUPPORTED
    assert comb(d=12) == ERR_UNSUPPORTED
    assert comb(out=5) == ERR_UNSUPPORTED
    assert comb(yp=None) == ERR_NULL
    assert comb(y=FAKE + 4) == ERR_ALIGN
    assert comb(T=0, yp=None, y=None) == 0


def test_combine_backward_validation(L):
    def cb(T=4, d=64, k=2, rows=8, dy=FAKE, yp=FAKE, dyp=FAKE, dw=FAKE):
        return L.moe_combine_backward(dy, yp, FAKE, FAKE, T, d, k, rows, dyp, dw, None)
    assert cb(k=0) == ERR_SHAPE
    assert cb(rows=-1) == ERR_SHAPE
    assert cb(k=9) == ERR_UNSUPPORTED
    assert cb(d=12) == ERR_UNSUPPORTED
    assert cb(dy=None) == ERR_NULL
    assert cb(yp=None) == ERR_NULL
    assert cb(dyp=None) == ERR_NULL
    assert cb(dw=None) == ERR_NULL
    assert cb(dy=FAKE + 4) == ERR_ALIGN
    assert cb(dyp=FAKE + 8) == ERR_ALIGN
    assert cb(T=0, dy=None, yp=None, dyp=None, dw=None) == 0


def test_grouped_gemm_packed_validation(L):
    def gg(G=2, rows=8, K=64, N=64, a=FAKE, w=FAKE, out=FAKE):
        return L.moe_grouped_gemm_packed(a, FAKE, G, rows, K, N, w, out, None)
    assert gg(G=0) == ERR_SHAPE
    assert gg(rows=-1) == ERR_SHAPE
    assert gg(K=32) == ERR_SHAPE
    assert gg(K=96) == ERR_UNSUPPORTED
    assert gg(N=100) == ERR_UNSUPPORTED
    assert gg(K=4194240 + 64) == ERR_UNSUPPORTED   # one weight panel past 2 GiB
    assert gg(G=5000) == ERR_UNSUPPORTED
    assert gg(a=None) == ERR_NULL
    assert gg(w=None) == ERR_NULL
    assert gg(out=FAKE + 4) == ERR_ALIGN
    assert gg(rows=0, a=None, w=None, out=None) == 0


def test_swiglu_backward_validation(L):
    def sb(n=64, lim=10.0, mode=0, g=FAKE, dg=FAKE):
        return L.moe_swiglu_backward(g, FAKE, FAKE, n, ctypes.c_float(lim), mode, dg, FAKE, None)
    assert sb(n=-4) == ERR_SHAPE
    assert sb(n=6) == ERR_UNSUPPORTED
    assert sb(lim=0.0) == ERR_SHAPE
    assert sb(lim=float("nan")) == ERR_SHAPE
    assert sb(mode=2) == ERR_UNSUPPORTED
    assert sb(g=None) == ERR_NULL
    assert sb(dg=None) == ERR_NULL
    assert sb(g=FAKE + 4) == ERR_ALIGN
    assert sb(n=0, g=None, dg=None) == 0


def test_forward_validation(L):
    cfg = ops.MoeCfg(T=8, d=128, E=8, k=2, F=64, F_shared=64, mode=0, n_bias=1, V=0, scale=1.0,
                     clamp_limit=10.0, clamp_mode=0, out_dtype=0)
    w = ops.MoeWeights(packed=0, w_g=FAKE, logit_offset=None, score_bias=FAKE, tid2eid=None, w_gate=FAKE,
                       w_up=FAKE, w_down=FAKE, s_gate=FAKE, s_up=FAKE, s_down=FAKE)
    need = L.moe_forward_workspace_size(ctypes.byref(cfg))
    assert need > 0

    def fwd(c=cfg, wt=w, x=FAKE, ws=FAKE, wsb=need, ids=None):
        return L.moe_forward(ctypes.byref(c), ctypes.byref(wt), x, ids, None, FAKE, None, None,
                             None, None, ws, wsb, None)
    assert L.moe_forward(None, ctypes.byref(w), FAKE, None, None, FAKE, None, None, None, None,
                         FAKE, need, None) == ERR_NULL
    assert fwd(x=None) == ERR_NULL
    assert fwd(ws=None) == ERR_NULL
    assert fwd(wsb=need - 1) == ERR_WORKSPACE
    assert fwd(x=FAKE + 2) == ERR_ALIGN
    for field, val, code in (("k", 9, ERR_UNSUPPORTED), ("k", 0, ERR_SHAPE),
                             ("d", 100, ERR_UNSUPPORTED), ("F_shared", 32, ERR_UNSUPPORTED),
                             ("mode", 3, ERR_UNSUPPORTED), ("out_dtype", 2, ERR_UNSUPPORTED),
                             ("clamp_limit", -1.0, ERR_SHAPE), ("E", 4096, ERR_UNSUPPORTED)):
        c = ops.MoeCfg.from_buffer_copy(cfg)
        setattr(c, field, val)
        assert fwd(c=c) == code, field
    wp = ops.MoeWeights.from_buffer_copy(w)
    wp.packed = 5
    assert fwd(wt=wp) == ERR_UNSUPPORTED
    wp.packed = ops.WEIGHTS_A8W4                     # A8W4 needs d and F multiples of 128
    assert fwd(wt=wp) == ERR_UNSUPPORTED
    c8 = ops.MoeCfg.from_buffer_copy(cfg)
    c8.F = 128
    need8 = L.moe_forward_workspace_size(ctypes.byref(c8))
    assert fwd(c=c8, wt=wp, wsb=need8) == ERR_NULL   # ... and the MXFP4 block scales
    wp.packed = ops.WEIGHTS_FP4                      # MXFP4 weights need their block scales
    assert fwd(wt=wp) == ERR_NULL
    wp.packed = ops.WEIGHTS_FP8                      # MXFP8 weights need their block scales
    assert fwd(wt=wp) == ERR_NULL
    wp.w_gate_scale = wp.w_up_scale = wp.w_down_scale = FAKE + 4
    assert fwd(wt=wp) == ERR_ALIGN
    c = ops.MoeCfg.from_buffer_copy(cfg)
    c.mode = 1
    c.V = 100
    assert fwd(c=c) == ERR_NULL                      # hash mode needs input_ids + tid2eid
    c.T = 0
    assert fwd(c=c, x=None, ws=None) == 0
    c = ops.MoeCfg.from_buffer_copy(cfg)
    c.T = 1 << 30                                    # T k = 2^31 routed rows: out of range
    assert fwd(c=c) == ERR_SHAPE


def test_workspace_size_and_error_flag_reader(L):
    """moe_workspace_size is the forward's workspace under the layer's one
    name (0 for an invalid cfg); moe_read_error_flags rejects NULL pointers
    before any HIP call."""
    cfg = ops.MoeCfg(T=8192, d=4096, E=384, k=6, F=2048, F_shared=2048, mode=0, n_bias=1, V=0,
                     scale=2.5, clamp_limit=10.0, clamp_mode=0, out_dtype=0)
    a = L.moe_workspace_size(ctypes.byref(cfg))
    assert a == L.moe_forward_workspace_size(ctypes.byref(cfg)) and a > 0
    assert L.moe_workspace_size(None) == 0
    bad = ops.MoeCfg.from_buffer_copy(cfg)
    bad.k = 0
    assert L.moe_workspace_size(ctypes.byref(bad)) == 0
    out = ctypes.c_uint32(7)
    assert L.moe_read_error_flags(None, None, ctypes.byref(out)) == ERR_NULL
    assert L.moe_read_error_flags(FAKE, None, None) == ERR_NULL
    assert out.value == 7


def test_permute_noalloc_validation(L):
    """moe_permute_noalloc: moe_permute's checks, and a call whose scratch
    exceeds the static array is rejected before any launch."""
    def pn(T=64, d=64, E=8, k=2, ids=FAKE, x=FAKE, counts=FAKE, offsets=FAKE, xp=FAKE):
        return L.moe_permute_noalloc(ids, x, T, d, E, k, counts, offsets, FAKE, FAKE, xp, None,
                                     None)
    assert pn(k=0) == ERR_SHAPE
    assert pn(E=2000) == ERR_UNSUPPORTED
    assert pn(d=12) == ERR_UNSUPPORTED
    assert pn(counts=None) == ERR_NULL
    assert pn(ids=None) == ERR_NULL
    assert pn(x=FAKE + 2) == ERR_ALIGN
    T, k, E = 1 << 18, 8, 1024                # entry ranks alone: 8 MiB
    assert ops.permute_workspace_size(T, k, E) > 8 << 20
    assert pn(T=T, k=k, E=E) == -7
    assert "scratch" in L.moe_status_string(-7).decode()


def test_grouped_wgrad_validation(L):
    def wg(G=2, rows=64, M=64, K=64, dy=FAKE, a=FAKE, offs=FAKE, dw=FAKE):
        return L.moe_grouped_wgrad(dy, a, offs, G, rows, M, K, dw, None)
    assert wg(G=0) == ERR_SHAPE
    assert wg(rows=-1) == ERR_SHAPE
    assert wg(M=4) == ERR_SHAPE
    assert wg(M=68) == ERR_UNSUPPORTED
    assert wg(K=100) == ERR_UNSUPPORTED
    assert wg(dw=None) == ERR_NULL
    assert wg(dy=None) == ERR_NULL
    assert wg(offs=None) == ERR_NULL                 # several groups need offsets
    assert wg(a=FAKE + 8) == ERR_ALIGN
    assert wg(G=1 << 20, M=4096, K=4096) == ERR_SHAPE
