"""Helpers shared by the GPU parity tests: host copies for the oracle and the
tolerances the tests apply.

Tolerances (fp32 accumulation of bf16 products, no other rounding):
  - router logits: |l_gpu - l_ref| <= 2 * d * 2^-24 * sum_i |x_i w_i|  (a
    worst-case bound for any summation order of d terms, plus the rounding of
    the offset add) - l_ref from the fp64 oracle;
  - h (bf16): |h_gpu - h_ref| <= ulp_bf16(h_ref) + |dh|, where dh bounds the
    fp32 pre-activation error: |dh| <= 1.1 |U| dG + |silu(G)| dU + 2^-18 |h|
    with dG, dU <= 2 d 2^-24 sum_i |a_i w_i| (fp32 accumulation, any order;
    1.1 bounds |silu'|, the clamp is 1-Lipschitz); both sides round once to
    bf16, so they differ by at most the pre-rounding error plus one ulp.  G
    and U for the bound come from numpy fp64 matmuls;
  - y, y_perm: max |y - y_ref| <= 1e-2 * RMS(y_ref), the acceptance bar.
"""
import numpy as np
import torch

import oracle
from sparse_moe_layer_04_amd import workloads as wl

bits = wl.bf16_bits


def host(t):
    return t.detach().cpu().numpy()


def bf16_f64(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def check_logits(x_bits, wg_bits, off, got, rows=None):
    """Compare GPU logits (rows subset) against the oracle's fp64 logits."""
    if rows is None:
        rows = np.arange(x_bits.shape[0])
    xs = x_bits[rows]
    ref = oracle.gate_logits(xs, wg_bits, off).astype(np.float64)
    mag = np.abs(bf16_f64(xs)) @ np.abs(bf16_f64(wg_bits)).T
    d = x_bits.shape[1]
    bound = 2 * d * 2.0 ** -24 * mag + np.abs(ref) * 2.0 ** -23
    err = np.abs(got[rows].astype(np.float64) - ref)
    assert np.all(err <= bound), float((err / np.maximum(bound, 1e-30)).max())
    return float(err.max())


def h_bound(a_bits, wg_bits, wu_bits, L, mode):
    """Allowed |h_gpu - h_ref| beyond one bf16 ulp for rows a through one
    expert's gate/up weights (see the module docstring)."""
    a = bf16_f64(a_bits)
    wg = bf16_f64(wg_bits)
    wu = bf16_f64(wu_bits)
    G = a @ wg.T
    U = a @ wu.T
    d = a.shape[1]
    dG = 2 * d * 2.0 ** -24 * (np.abs(a) @ np.abs(wg).T)
    dU = 2 * d * 2.0 ** -24 * (np.abs(a) @ np.abs(wu).T)
    G = np.minimum(np.maximum(G, -L), L) if mode == 0 else np.minimum(G, L)
    U = np.minimum(np.maximum(U, -L), L)
    with np.errstate(over="ignore"):
        silu = G / (1 + np.exp(-G))
    return 1.1 * np.abs(U) * dG + np.abs(silu) * dU + 2.0 ** -18 * np.abs(silu * U)


def check_h(h_gpu_bits, h_ref_bits, bound):
    a = bf16_f64(h_gpu_bits)
    b = bf16_f64(h_ref_bits)
    bad = a != b
    frac = float(bad.mean()) if bad.size else 0.0
    if bad.any():
        ulp = np.spacing(np.abs(b).astype(np.float32)).astype(np.float64) * 2.0 ** 16
        ulp = np.maximum(ulp, 2.0 ** -133)
        excess = np.abs(a - b) - ulp * 1.0001 - bound
        assert np.all(excess[bad] <= 0), f"h beyond bound at {np.argwhere(excess > 0)[:5]}"
    assert frac <= 5e-3, f"{frac:.4%} of h differ"
    return frac


def ffn_h_bound(a_bits, offsets, wg_bits, wu_bits, L, mode):
    """h_bound for a grouped FFN (rows of group g through expert g)."""
    out = np.zeros((a_bits.shape[0], wg_bits.shape[1]))
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            out[lo:hi] = h_bound(a_bits[lo:hi], wg_bits[g], wu_bits[g], L, mode)
    return out


def check_rms(got, ref, tol=1e-2):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert err <= tol * rms + 1e-30, f"max err {err:.3e} > {tol} * rms {rms:.3e}"
    return err / rms if rms else 0.0


def near_ties(logits, bias_rows, k, gap=1e-6):
    """Tokens whose k-th and (k+1)-th biased scores differ by less than `gap`
    (scores from the oracle's binary32 sigmoid)."""
    s = oracle.score(logits)
    r = (s + bias_rows).astype(np.float64) if bias_rows is not None else s.astype(np.float64)
    if r.shape[1] <= k:
        return 0
    part = -np.sort(-r, axis=1)[:, k - 1:k + 1]
    return int((part[:, 0] - part[:, 1] < gap).sum())


def route_flips(xb, wg, off, lg_gpu, bias, modality, ids_gpu, k):
    """TopK route flips between the oracle's fp64-accumulated logits and the
    GPU's fp32 logits: [(token, gap, bound)] for every token whose expert set
    differs.  gap = k-th minus (k+1)-th biased score under the GPU logits;
    bound = 0.5 x max |logit difference| of the row + 1e-6 (sigmoid slope is
    at most 1/4, and the two scores of the swapped pair can both move)."""
    lg_ref = oracle.gate_logits(xb, wg, off)
    ids_ref, _, _ = oracle.route(lg_ref, k, 1.0, bias=bias, modality=modality)
    rows = 0.0
    if bias is not None:
        b = np.asarray(bias, np.float64).reshape(-1, lg_gpu.shape[1])
        rows = b[modality.astype(np.int64)] if (modality is not None and b.shape[0] > 1) else b[:1]
    r_gpu = oracle.score(lg_gpu).astype(np.float64) + rows
    diff = np.abs(lg_ref.astype(np.float64) - lg_gpu.astype(np.float64)).max(axis=1)
    out = []
    for t in np.nonzero(np.any(np.sort(ids_ref, axis=1) != np.sort(ids_gpu, axis=1), axis=1))[0]:
        part = -np.sort(-r_gpu[t])[k - 1:k + 1]
        out.append((int(t), float(part[0] - part[1]), float(0.5 * diff[t] + 1e-6)))
    return out


def free_cuda():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def case_id(w):
    """pytest id of a workload case: its name, seed and any non-default clamp."""
    s = f"{w.name}-s{w.seed}"
    if w.clamp_limit != 10.0 or w.clamp_mode != 0:
        s += f"-L{w.clamp_limit:g}-m{w.clamp_mode}"
    return s
