"""Seeded synthetic inputs shaped like DeepSeek-V3's FP8 projections.

This module only draws random numbers and arranges them; it holds none of the
quantized linear path's arithmetic (no act_quant, no dequant, no GEMM), so the
CPU oracle and the GPU library can both be fed from it.

Recipe (each choice is also listed in the design notes):

* seeds: ``1000 * config + tensor_id`` on a CPU ``torch.Generator``; tensor ids
  0 = x, 1 = W1 values, 2 = W1 scales, 3 = W2 values, 4 = W2 scales,
  5 = outlier mask, 6 = routing scores, 7 = W3 values, 8 = W3 scales;
* activations: float32 N(0,1), optionally with a Bernoulli(p) mask of entries
  multiplied by an outlier factor, then rounded to bf16 by torch;
* weight scales: ``2**U`` with U uniform on ``[lo, hi]`` (log-uniform), fp32,
  one per 128x128 block;
* weight codes: the offline checkpoint's quantization is stood in for by
  torch's own ``float8_e4m3fn`` cast of ``N(0,1) / scale`` clamped to +-448
  (torch's cast rounds to nearest-even; the clamp makes it saturate);
* routing: per token, 256 uniform scores; a stable descending sort picks the
  top 8 (ties to the lower expert id); the routing weights are the chosen
  scores over their sum; experts 0..31 are the local ones, each with its
  tokens in ascending order.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

BLOCK = 128

# dims of the DeepSeek-V3 projections the workloads are shaped like
DIM = 7168
MOE_INTER = 2048
DENSE_INTER = 18432
Q_LORA_RANK = 1536
N_ROUTED = 256
TOP_K = 8
LOCAL_EXPERTS = 32


def seed_of(config: int, tensor_id: int) -> int:
    return 1000 * config + tensor_id


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def activations(M: int, K: int, seed: int, outlier_p: float = 0.0,
                outlier_factor: float = 20.0, outlier_seed: Optional[int] = None) -> torch.Tensor:
    """bf16 [M, K] drawn from N(0,1); a Bernoulli(outlier_p) subset is scaled up."""
    x = torch.randn(M, K, generator=_gen(seed), dtype=torch.float32)
    if outlier_p > 0.0:
        u = torch.rand(M, K, generator=_gen(outlier_seed if outlier_seed is not None else seed + 5),
                       dtype=torch.float32)
        x = torch.where(u < outlier_p, x * outlier_factor, x)
    return x.to(torch.bfloat16)


def block_scales(n_blocks: int, k_blocks: int, seed: int, lo: float = -8.0,
                 hi: float = -2.0) -> torch.Tensor:
    """fp32 [n_blocks, k_blocks] scales, log-uniform in [2**lo, 2**hi]."""
    u = torch.rand(n_blocks, k_blocks, generator=_gen(seed), dtype=torch.float64)
    return torch.exp2(lo + (hi - lo) * u).to(torch.float32)


def weight_codes(N: int, K: int, scales: torch.Tensor, seed: int) -> torch.Tensor:
    """uint8 [N, K] e4m3 codes standing for a checkpoint weight quantized with ``scales``."""
    w = torch.randn(N, K, generator=_gen(seed), dtype=torch.float32)
    expanded = scales.repeat_interleave(BLOCK, 0)[:N].repeat_interleave(BLOCK, 1)[:, :K]
    v = torch.clamp(w / expanded, -448.0, 448.0)
    return v.to(torch.float8_e4m3fn).view(torch.uint8)


def weight(N: int, K: int, value_seed: int, scale_seed: int, lo: float = -8.0,
           hi: float = -2.0, pow2: bool = False):
    """(codes uint8 [N,K], scales fp32 [ceil(N/128), ceil(K/128)]).

    pow2: the scales are rounded to the nearest power of two (a checkpoint with
    power-of-two block scales)."""
    S = block_scales(-(-N // BLOCK), -(-K // BLOCK), scale_seed, lo, hi)
    if pow2:
        S = torch.exp2(torch.round(torch.log2(S.double()))).to(torch.float32)
    return weight_codes(N, K, S, value_seed), S


def routing_table(tokens: int, seed: int, n_experts: int = N_ROUTED, top_k: int = TOP_K):
    """(topk int32 [tokens, top_k], weights fp32 [tokens, top_k]).

    Per token, n_experts uniform scores stand in for the gate's sigmoid scores;
    a stable descending sort picks the top_k experts (ties to the lower id), and
    the weights are the chosen scores divided by their sum (route scale 1).
    """
    scores = torch.rand(tokens, n_experts, generator=_gen(seed), dtype=torch.float32)
    top = torch.sort(scores, dim=1, descending=True, stable=True)
    idx = top.indices[:, :top_k].to(torch.int32).contiguous()
    val = top.values[:, :top_k]
    weights = (val / val.sum(dim=1, keepdim=True)).to(torch.float32).contiguous()
    return idx, weights


def routing(tokens: int, seed: int, n_experts: int = N_ROUTED, top_k: int = TOP_K,
            local: int = LOCAL_EXPERTS):
    """Token ids grouped by local expert (experts 0 .. local-1), and int32 offsets [local+1]."""
    order, _ = routing_table(tokens, seed, n_experts, top_k)
    ids: List[torch.Tensor] = []
    counts = []
    for e in range(local):
        hit = (order == e).any(dim=1).nonzero(as_tuple=False).flatten()
        ids.append(hit)
        counts.append(hit.numel())
    token_ids = torch.cat(ids).to(torch.int64)
    offsets = torch.zeros(local + 1, dtype=torch.int32)
    offsets[1:] = torch.cumsum(torch.tensor(counts, dtype=torch.int64), 0).to(torch.int32)
    return token_ids, offsets


@dataclass
class Workload:
    """One named configuration: its tensors (CPU) and the GEMM shapes it runs."""
    name: str
    config: int
    tensors: Dict[str, torch.Tensor] = field(default_factory=dict)
    meta: Dict[str, object] = field(default_factory=dict)


WORKLOAD_NAMES = {
    0: "tiny-linear-16x256x256",
    1: "decode-q-down-64x1536x7168",
    2: "prefill-moe-expert-pair-4096x7168x2048",
    3: "dense-mlp-layer0-8192x18432x7168",
    4: "grouped-routed-experts-32of256-top8-8192tok",
}


def make(config: int, scale: float = 1.0) -> Workload:
    """Build configuration ``config`` (0..4).  ``scale`` < 1 shrinks M (tests only)."""
    wl = Workload(WORKLOAD_NAMES[config], config)
    t = wl.tensors
    if config == 0:
        M, N, K = 16, 256, 256
        t["x"] = activations(M, K, seed_of(0, 0))
        t["w1"], t["s1"] = weight(N, K, seed_of(0, 1), seed_of(0, 2), -8.0, -2.0)
        wl.meta.update(M=M, N=N, K=K)
    elif config == 1:
        M, N, K = 64, Q_LORA_RANK, DIM
        t["x"] = activations(M, K, seed_of(1, 0), outlier_p=0.01, outlier_factor=20.0,
                             outlier_seed=seed_of(1, 5))
        t["w1"], t["s1"] = weight(N, K, seed_of(1, 1), seed_of(1, 2), -10.0, -4.0)
        wl.meta.update(M=M, N=N, K=K)
    elif config == 2:
        M = max(1, int(4096 * scale))
        t["x"] = activations(M, DIM, seed_of(2, 0))
        t["w1"], t["s1"] = weight(MOE_INTER, DIM, seed_of(2, 1), seed_of(2, 2))
        t["w2"], t["s2"] = weight(DIM, MOE_INTER, seed_of(2, 3), seed_of(2, 4))
        # the gated expert's third projection (w3), for the fused gated-FFN step
        t["w3"], t["s3"] = weight(MOE_INTER, DIM, seed_of(2, 7), seed_of(2, 8))
        wl.meta.update(M=M, N1=MOE_INTER, K1=DIM, N2=DIM, K2=MOE_INTER)
    elif config == 3:
        M = max(1, int(8192 * scale))
        t["x"] = activations(M, DIM, seed_of(3, 0))
        t["w1"], t["s1"] = weight(DENSE_INTER, DIM, seed_of(3, 1), seed_of(3, 2))
        t["w2"], t["s2"] = weight(DIM, DENSE_INTER, seed_of(3, 3), seed_of(3, 4))
        wl.meta.update(M=M, N1=DENSE_INTER, K1=DIM, N2=DIM, K2=DENSE_INTER)
    elif config == 4:
        tokens = max(1, int(8192 * scale))
        t["x"] = activations(tokens, DIM, seed_of(4, 0))
        token_ids, offsets = routing(tokens, seed_of(4, 6))
        t["token_ids"], t["offsets"] = token_ids, offsets
        t["topk"], t["weights"] = routing_table(tokens, seed_of(4, 6))
        G = LOCAL_EXPERTS
        codes = torch.empty(G, MOE_INTER, DIM, dtype=torch.uint8)
        scales = torch.empty(G, MOE_INTER // BLOCK, DIM // BLOCK, dtype=torch.float32)
        for g in range(G):
            # one value stream and one scale stream per expert, derived from the config seeds
            codes[g], scales[g] = weight(MOE_INTER, DIM, seed_of(4, 1) * 100 + g,
                                         seed_of(4, 2) * 100 + g)
        t["w1"], t["s1"] = codes, scales
        wl.meta.update(tokens=tokens, T=int(offsets[-1]), G=G, N=MOE_INTER, K=DIM)
    else:
        raise ValueError(f"unknown configuration {config}")
    return wl
