"""Seeded synthetic workloads for MoE token dispatch and combine.

Every input is synthetic.  The pages describe the problem shapes (top-k routing
with -1 meaning unrouted, fp32 top-k weights, bf16 hidden rows) but ship no
dataset, so the arrays below stand in for a router's output:

* hidden rows ``x``: i.i.d. N(0, 1) drawn in float32, rounded to bf16 by torch
  (a library conversion, so this module carries no rounding code of its own);
* top-k ids: ``K`` distinct experts per token, either uniform over the ``E``
  experts or Zipf(s) over a random permutation of the experts (Gumbel top-k,
  i.e. sequential sampling without replacement);
* top-k weights: softmax of N(0, 1) logits over the K slots, in float64,
  then cast to float32; optionally a fraction of slots is set to -1 (unrouted)
  with weight 0 and the remaining weights are renormalised.

Four independent PCG64 streams (hidden rows, ids, logits, unrouted mask) are
derived from one seed, so routing can be drawn without materialising ``x`` and the first
``n`` tokens of a workload equal the workload drawn with ``T = n``.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "WorkloadSpec",
    "Workload",
    "CONFIGS",
    "spec",
    "make_routing",
    "make_hidden",
    "make_workload",
    "balanced_routing",
]


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    T: int                      # tokens
    H: int                      # hidden size (bf16 channels)
    E: int                      # global experts
    K: int                      # top-k slots per token
    P: int                      # destinations (EP ranks); E = P * E_local
    routing: str = "uniform"    # "uniform" | "zipf"
    zipf_s: float = 1.2
    unrouted_frac: float = 0.0  # fraction of slots forced to -1
    layout: str = "send"        # "send" (destination-major) | "batched" | "expert_major"
    first_expert: int = 0       # batched layout: first local expert
    max_num_tokens: int = 0     # batched layout: rows per local expert
    fp8: bool = False           # quantise rows to e4m3 on dispatch
    scale_fmt: str = "f32"      # fp8 scales: "f32", "pow2" or "ue8m0"
    scale_col_major: bool = False  # batched fp8: scales column-major per expert
    align: int = 1              # expert-major layout: rows per expert padded to a multiple
    chunks: int = 1             # contiguous token chunks
    streams: int = 1            # HIP streams the chunks alternate over
    seed: int = 0

    @property
    def E_local(self) -> int:
        return self.E // self.P

    def replace(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)


# The five workloads the dispatch/combine path is sized for.
CONFIGS = {
    "tiny": WorkloadSpec("tiny", T=256, H=512, E=8, K=2, P=2),
    "uniform_t4096": WorkloadSpec("uniform_t4096", T=4096, H=4096, E=64, K=6, P=8),
    "batched_t8192": WorkloadSpec(
        "batched_t8192", T=8192, H=7168, E=256, K=8, P=8, layout="batched",
        first_expert=0, max_num_tokens=8192),
    "batched_fp8_t8192": WorkloadSpec(
        "batched_fp8_t8192", T=8192, H=7168, E=256, K=8, P=8, layout="batched",
        first_expert=0, max_num_tokens=8192, fp8=True, scale_fmt="ue8m0",
        scale_col_major=True),
    "skewed_t16384": WorkloadSpec(
        "skewed_t16384", T=16384, H=7168, E=256, K=8, P=32, routing="zipf",
        zipf_s=1.2, unrouted_frac=0.05),
    "expert_major_t16384": WorkloadSpec(
        "expert_major_t16384", T=16384, H=7168, E=256, K=8, P=32, routing="zipf",
        zipf_s=1.2, unrouted_frac=0.05, layout="expert_major", align=128),
    "fp8_t32768": WorkloadSpec(
        "fp8_t32768", T=32768, H=7168, E=256, K=8, P=32, fp8=True, chunks=4,
        streams=1),     # the pipelined 2-stream schedule: streams=2
}


def spec(name: str, **overrides) -> WorkloadSpec:
    s = CONFIGS[name]
    return s.replace(**overrides) if overrides else s


@dataclasses.dataclass
class Workload:
    spec: WorkloadSpec
    topk_idx: np.ndarray               # int64 [T, K], -1 = unrouted
    topk_weights: np.ndarray           # float32 [T, K]
    x_bits: Optional[np.ndarray]       # uint16 [T, H] bf16 bit patterns


def _streams(seed: int):
    ss = np.random.SeedSequence(int(seed))
    kids = ss.spawn(4)
    return [np.random.Generator(np.random.PCG64(k)) for k in kids]


def make_routing(s: WorkloadSpec):
    """Return (topk_idx int64 [T,K], topk_weights float32 [T,K])."""
    _, g_ids, g_w, g_mask = _streams(s.seed)
    T, E, K = s.T, s.E, s.K
    if K > E:
        raise ValueError("K must not exceed E")
    if s.routing == "uniform":
        keys = g_ids.random((T, E))
        ids = np.argsort(keys, axis=1, kind="stable")[:, :K]
    elif s.routing == "zipf":
        perm = g_ids.permutation(E)
        p = np.empty(E, dtype=np.float64)
        p[perm] = (np.arange(E, dtype=np.float64) + 1.0) ** (-s.zipf_s)
        p /= p.sum()
        keys = np.log(p)[None, :] + g_ids.gumbel(size=(T, E))
        ids = np.argsort(-keys, axis=1, kind="stable")[:, :K]
    else:
        raise ValueError(f"unknown routing {s.routing!r}")
    ids = np.ascontiguousarray(ids.astype(np.int64))

    logits = g_w.standard_normal((T, K))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    if s.unrouted_frac > 0.0:
        mask = g_mask.random((T, K)) < s.unrouted_frac
        ids[mask] = -1
        w[mask] = 0.0
        tot = w.sum(axis=1, keepdims=True)
        np.divide(w, tot, out=w, where=tot > 0)
    return ids, np.ascontiguousarray(w.astype(np.float32))


def make_hidden(s: WorkloadSpec, rows: Optional[int] = None) -> np.ndarray:
    """bf16 bit patterns (uint16 [rows, H]) of N(0,1) hidden rows."""
    import torch

    g_x = _streams(s.seed)[0]
    n = s.T if rows is None else int(rows)
    out = np.empty((n, s.H), dtype=np.uint16)
    step = max(1, (1 << 24) // max(1, s.H))       # rows per block (~64 MB f32)
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        blk = g_x.standard_normal((r1 - r0, s.H), dtype=np.float32)
        out[r0:r1] = (torch.from_numpy(blk).to(torch.bfloat16)
                      .view(torch.int16).numpy().view(np.uint16))
    return out


def make_workload(s: WorkloadSpec, with_x: bool = True) -> Workload:
    ids, w = make_routing(s)
    x = make_hidden(s) if with_x else None
    return Workload(spec=s, topk_idx=ids, topk_weights=w, x_bits=x)


def balanced_routing(T: int, K: int, E: int):
    """Forced-balanced routing: slot k of token t picks expert (t*K + k) mod E.

    This is the benchmark-only static routing of the NeMo token dispatcher
    (TokenDispatcherConfig, moe_benchmark_static_routing): every expert gets
    the same number of slots when E divides T*K.  Weights are uniform 1/K.
    """
    t = np.arange(T, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    ids = (t * K + k) % E
    w = np.full((T, K), 1.0 / K, dtype=np.float32)
    return ids, w
