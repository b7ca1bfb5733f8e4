"""Seeded synthetic workloads for the MoE layer forward.

This module only draws inputs: it holds none of the layer's arithmetic and is
the one piece shared by the HIP path's callers (tests, bench) and the oracle's
callers.  Every tensor is drawn from its own torch generator (or numpy
Generator for the integer streams), seeded from the workload seed and the
tensor's name, so a workload is reproducible on a given device.

Shapes follow the pages' layer (384 routed experts, top-6, one shared expert:
"MindSpore HyperParallel one-click DeepSeek-V4.1-Flash", section 01) and the
five workload definitions below; distributions:
  x ~ N(0,1); router / expert / shared weights ~ N(0, std = 1/sqrt(fan_in))
  (fan_in = d for W_g, W_gate, W_up; F for W_down), all rounded to bf16;
  routing bias ~ U(-0.1, 0.1) fp32 (one vector, or text + vision vectors);
  skewed workload: 4 contiguous 576-token image spans and a per-expert logit
  offset ln(E * p_e) with p_e proportional to rank_e^-1.2 (Zipf popularity,
  ranks a seeded permutation of 1..E);
  hash workload: input_ids with P(id = r-1) proportional to r^-1.1 over the
  vocabulary, and a tid2eid table whose rows hold k distinct experts drawn
  uniformly at random.
"""
from dataclasses import dataclass, field
import hashlib
import math

import numpy as np
import torch

MODE_TOPK = 0
MODE_HASH = 1


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    scale: float
    seed: int
    mode: int = MODE_TOPK
    n_bias: int = 1
    F_shared: int = -1          # -1: same width as the routed experts; 0: no shared expert
    clamp_limit: float = 10.0
    clamp_mode: int = 0
    vision_spans: int = 0       # number of 576-token image spans (skewed workload)
    span_len: int = 576
    zipf_expert_s: float = 0.0  # > 0: Zipf(s) expert popularity as a logit offset
    V: int = 0                  # hash mode vocabulary
    zipf_token_s: float = 0.0   # hash mode input-id Zipf exponent
    extra: dict = field(default_factory=dict)

    @property
    def Fs(self) -> int:
        return self.F if self.F_shared < 0 else self.F_shared

    def describe(self) -> dict:
        out = dict(workload=self.name, T=self.T, d=self.d, E=self.E, k=self.k, F=self.F,
                   F_shared=self.Fs, scale=self.scale,
                   router="hash" if self.mode == MODE_HASH else "topk", n_bias=self.n_bias,
                   clamp_limit=self.clamp_limit, seed=self.seed)
        if self.vision_spans:
            out["vision_spans"] = self.vision_spans
        if self.zipf_expert_s:
            out["zipf_expert_s"] = self.zipf_expert_s
        if self.mode == MODE_HASH:
            out["V"] = self.V
            out["zipf_token_s"] = self.zipf_token_s
        return out


WORKLOADS = {
    0: Workload("tiny-T64-d128-E8-k2-F64", T=64, d=128, E=8, k=2, F=64, scale=1.0, seed=0),
    1: Workload("mid-T4096-d2048-E64-k6-F1024", T=4096, d=2048, E=64, k=6, F=1024,
                scale=1.0, seed=1),
    2: Workload("v4flash-T8192-d4096-E384-k6-F2048", T=8192, d=4096, E=384, k=6, F=2048,
                scale=2.5, seed=2),
    3: Workload("skewed-multimodal-T8192-d4096-E384-k6-F2048", T=8192, d=4096, E=384, k=6,
                F=2048, scale=2.5, seed=3, n_bias=2, vision_spans=4, zipf_expert_s=1.2),
    4: Workload("hash-T32768-d4096-E384-k6-F2048", T=32768, d=4096, E=384, k=6, F=2048,
                scale=2.5, seed=4, mode=MODE_HASH, V=129280, zipf_token_s=1.1),
}


def small(T, d, E, k, F, seed, scale=1.0, **kw) -> Workload:
    """An ad-hoc workload with the tiny workload's distributions."""
    return Workload(f"adhoc-T{T}-d{d}-E{E}-k{k}-F{F}", T=T, d=d, E=E, k=k, F=F,
                    scale=scale, seed=seed, **kw)


def _subseed(seed: int, name: str) -> int:
    h = hashlib.sha256(f"{seed}:{name}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 62) - 1)


def _gen(seed, name, device):
    g = torch.Generator(device=device)
    g.manual_seed(_subseed(seed, name))
    return g


def _normal_bf16(shape, std, seed, name, device, chunk_dim0=False):
    """N(0, std^2) drawn in fp32 and rounded to bf16 (RNE); optionally one
    generator call per leading index to bound the fp32 temporary."""
    g = _gen(seed, name, device)
    if not chunk_dim0:
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(torch.bfloat16)
    out = torch.empty(shape, device=device, dtype=torch.bfloat16)
    for i in range(shape[0]):
        t = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
        t.mul_(std)
        out[i].copy_(t)
    return out


def _uniform_f32(shape, lo, hi, seed, name, device):
    g = _gen(seed, name, device)
    t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def vision_mask(w: Workload) -> np.ndarray:
    """modality[T] u8: 1 inside `vision_spans` non-overlapping image spans."""
    rng = np.random.default_rng(_subseed(w.seed, "vision_spans"))
    slots = w.T // w.span_len
    starts = np.sort(rng.choice(slots, size=w.vision_spans, replace=False)) * w.span_len
    m = np.zeros(w.T, np.uint8)
    for s in starts:
        m[s:s + w.span_len] = 1
    return m


def zipf_logit_offset(w: Workload) -> np.ndarray:
    """offset_e = ln(E * p_e), p_e proportional to rank_e^-s, ranks permuted."""
    rng = np.random.default_rng(_subseed(w.seed, "zipf_expert"))
    ranks = rng.permutation(w.E) + 1
    p = ranks.astype(np.float64) ** (-w.zipf_expert_s)
    p /= p.sum()
    return np.log(w.E * p).astype(np.float32)


def zipf_input_ids(w: Workload) -> np.ndarray:
    rng = np.random.default_rng(_subseed(w.seed, "input_ids"))
    r = np.arange(1, w.V + 1, dtype=np.float64)
    p = r ** (-w.zipf_token_s)
    p /= p.sum()
    return rng.choice(w.V, size=w.T, p=p).astype(np.int32)


def hash_table(w: Workload) -> np.ndarray:
    """tid2eid[V, k]: each row k distinct experts, uniformly random (Floyd's
    subset sampling, then a uniform shuffle of the row)."""
    rng = np.random.default_rng(_subseed(w.seed, "tid2eid"))
    V, E, k = w.V, w.E, w.k
    tab = np.empty((V, k), np.int64)
    for j in range(k):
        top = E - k + j
        c = rng.integers(0, top + 1, size=V)
        dup = (tab[:, :j] == c[:, None]).any(axis=1) if j else np.zeros(V, bool)
        tab[:, j] = np.where(dup, top, c)
    tab = rng.permuted(tab, axis=1)
    return tab.astype(np.int32)


def make_inputs(w: Workload, device="cpu", with_experts=True) -> dict:
    """All layer inputs of workload `w` as torch tensors on `device`.

    Keys: x, w_g, logit_offset, score_bias, modality, input_ids, tid2eid,
    w_gate, w_up, w_down, s_gate, s_up, s_down (absent ones are None).
    """
    s = w.seed
    big = w.E * w.F * w.d > (1 << 24)
    out = dict(
        x=_normal_bf16((w.T, w.d), 1.0, s, "x", device),
        w_g=_normal_bf16((w.E, w.d), 1.0 / math.sqrt(w.d), s, "w_g", device),
        logit_offset=None, score_bias=None, modality=None, input_ids=None, tid2eid=None,
        w_gate=None, w_up=None, w_down=None, s_gate=None, s_up=None, s_down=None,
    )
    if w.mode == MODE_TOPK:
        out["score_bias"] = _uniform_f32((w.n_bias, w.E), -0.1, 0.1, s, "score_bias", device)
        if w.vision_spans:
            out["modality"] = torch.from_numpy(vision_mask(w)).to(device)
        if w.zipf_expert_s:
            out["logit_offset"] = torch.from_numpy(zipf_logit_offset(w)).to(device)
    else:
        out["input_ids"] = torch.from_numpy(zipf_input_ids(w)).to(device)
        out["tid2eid"] = torch.from_numpy(hash_table(w)).to(device)
    if with_experts:
        out["w_gate"] = _normal_bf16((w.E, w.F, w.d), 1.0 / math.sqrt(w.d), s, "w_gate",
                                     device, chunk_dim0=big)
        out["w_up"] = _normal_bf16((w.E, w.F, w.d), 1.0 / math.sqrt(w.d), s, "w_up",
                                   device, chunk_dim0=big)
        out["w_down"] = _normal_bf16((w.E, w.d, w.F), 1.0 / math.sqrt(w.F), s, "w_down",
                                     device, chunk_dim0=big)
        if w.Fs > 0:
            out["s_gate"] = _normal_bf16((w.Fs, w.d), 1.0 / math.sqrt(w.d), s, "s_gate", device)
            out["s_up"] = _normal_bf16((w.Fs, w.d), 1.0 / math.sqrt(w.d), s, "s_up", device)
            out["s_down"] = _normal_bf16((w.d, w.Fs), 1.0 / math.sqrt(w.Fs), s, "s_down",
                                         device)
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 bit pattern of a bf16 tensor (for the oracle)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
