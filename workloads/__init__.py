"""Seeded synthetic inputs for the grouped matmul.

This module only draws numbers.  It holds none of the grouped matmul's
arithmetic and imports neither the product package nor the oracle; both
sides are fed the very same tensors built here.

Workloads follow the shapes on the MaxText PR page "Megablox: transposed-RHS
gmm_v2 kernel for the backward dlhs" (Context: a 128-expert top-8 MoE, 16k
tokens x per-device batch 2 = 32768 tokens, so 262144 expert rows; expert
weights of 507,510,784 B = 128 x 1408 x 1408 bf16 for wi and 253,755,392 B =
128 x 1408 x 704 bf16 for wo).  No dataset or trained weight is involved;
random values of the stated distributions stand in for them.

Recipes:
  group sizes  a softmax router with Zipf(alpha) expert popularity: expert
               e has weight rank_e^-alpha (ranks a seeded permutation); each
               token adds Gumbel noise to the log-weights and takes the top-k
               experts; group_sizes[e] counts the choices.
  values       normal draws in float32, cast to bfloat16 by torch (nearest
               even), or quantised to e4m3fn in blocks of 128 along K by
               ``quantize_e4m3_blocks`` (scale = amax/448, values divided by
               the scale, clamped to +-448 and cast by torch).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch

E4M3_MAX = 448.0


@dataclasses.dataclass
class Case:
    name: str
    lhs: torch.Tensor
    rhs: torch.Tensor               # the rhs passed to gmm (the active shard)
    group_sizes: torch.Tensor       # int32 [G]
    group_offset: int = 0
    transpose_rhs: bool = False
    rhs_scale: Optional[torch.Tensor] = None
    rhs_bias: Optional[torch.Tensor] = None
    lhs_scale: Optional[torch.Tensor] = None
    out_dtype: torch.dtype = torch.bfloat16
    meta: Dict = dataclasses.field(default_factory=dict)

    @property
    def M(self):
        return self.lhs.shape[0]

    @property
    def K(self):
        return self.lhs.shape[1]

    @property
    def N(self):
        return self.rhs.shape[2] if self.transpose_rhs else self.rhs.shape[1]

    @property
    def num_active(self):
        return self.rhs.shape[0]

    def sizes_list(self):
        return [int(x) for x in self.group_sizes.cpu().tolist()]

    def active_rows(self):
        s = self.sizes_list()
        return sum(s[self.group_offset:self.group_offset + self.num_active])

    def nonempty_active_groups(self):
        s = self.sizes_list()
        return sum(1 for x in s[self.group_offset:self.group_offset + self.num_active] if x > 0)

    def flops(self):
        """2 * (active rows) * N * K: rows are counted, not padded tiles."""
        return 2 * self.active_rows() * self.N * self.K

    def algorithmic_bytes(self):
        """Bytes the operation must move once: lhs rows of active groups,
        weights / scales / biases of active non-empty groups, all M x N
        outputs (inactive rows are written as zeros) and the group sizes."""
        K, N = self.K, self.N
        b = self.active_rows() * K * self.lhs.element_size()
        nz = self.nonempty_active_groups()
        b += nz * N * K * self.rhs.element_size()
        if self.rhs_scale is not None:
            b += nz * self.rhs_scale.shape[1] * N * 4
        if self.rhs_bias is not None:
            b += nz * N * self.rhs_bias.element_size()
        if self.lhs_scale is not None:
            b += self.active_rows() * self.lhs_scale.shape[1] * 4
        b += self.M * N * torch.tensor([], dtype=self.out_dtype).element_size()
        b += self.group_sizes.numel() * 4
        return b

    def to(self, device):
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return dataclasses.replace(self, lhs=mv(self.lhs), rhs=mv(self.rhs),
                                   group_sizes=mv(self.group_sizes),
                                   rhs_scale=mv(self.rhs_scale), rhs_bias=mv(self.rhs_bias),
                                   lhs_scale=mv(self.lhs_scale))


# ----------------------------------------------------------------------------
# group sizes


def router_group_sizes(seed: int, tokens: int, experts: int, top_k: int,
                       alpha: float = 1.1, forced_empty: int = 0) -> np.ndarray:
    """Counts of a Gumbel-top-k router over Zipf(alpha) expert popularity.

    ``forced_empty`` experts (a seeded choice) are removed before routing and
    stay at 0."""
    ss = np.random.SeedSequence(seed)
    r_empty, r_rank, r_gumbel = [np.random.default_rng(s) for s in ss.spawn(3)]
    live = np.ones(experts, dtype=bool)
    if forced_empty:
        live[r_empty.choice(experts, size=forced_empty, replace=False)] = False
    live_ids = np.nonzero(live)[0]
    n_live = live_ids.size
    if top_k > n_live:
        raise ValueError("top_k larger than the number of live experts")
    ranks = r_rank.permutation(n_live) + 1
    logw = -alpha * np.log(ranks.astype(np.float64))
    counts = np.zeros(experts, dtype=np.int64)
    chunk = 8192
    for t0 in range(0, tokens, chunk):
        t1 = min(tokens, t0 + chunk)
        g = r_gumbel.gumbel(size=(t1 - t0, n_live))
        choice = np.argpartition(-(logw[None, :] + g), top_k - 1, axis=1)[:, :top_k]
        counts[live_ids] += np.bincount(choice.ravel(), minlength=n_live)
    return counts.astype(np.int32)


def multinomial_group_sizes(seed: int, total: int, groups: int, empty=()) -> np.ndarray:
    """``total`` rows split Multinomial(total, uniform) over the groups not
    listed in ``empty``."""
    rng = np.random.default_rng(seed)
    live = [g for g in range(groups) if g not in set(empty)]
    draw = rng.multinomial(total, [1.0 / len(live)] * len(live))
    sizes = np.zeros(groups, dtype=np.int32)
    sizes[live] = draw
    return sizes


# ----------------------------------------------------------------------------
# values


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std: float, seed: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    t = torch.randn(*shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def quantize_e4m3_blocks(x: torch.Tensor, block: int = 128):
    """Quantise float32 x [..., K] to e4m3fn in blocks of ``block`` along the
    last axis.  Returns (q [..., K] e4m3fn, scale [..., K/block] float32) with
    x ~= q * scale per block; scale = amax/448 (1 for an all-zero block)."""
    K = x.shape[-1]
    if K % block:
        raise ValueError("K must be a multiple of the block")
    xb = x.reshape(*x.shape[:-1], K // block, block)
    amax = xb.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (xb / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.reshape(x.shape), scale.squeeze(-1).contiguous()


def _quantized_weight(G, N, K, std, seed, device, block=128):
    """W [G,N,K] normal(std) -> (e4m3 [G,N,K], rhs_scale [G,K/block,1,N])."""
    w = normal((G, N, K), std, seed, device)
    q, sc = quantize_e4m3_blocks(w, block)          # sc [G, N, nb]
    del w
    return q, sc.permute(0, 2, 1).unsqueeze(2).contiguous()


# ----------------------------------------------------------------------------
# the named workloads


def tiny_fp32(seed: int = 1001, device="cpu") -> Case:
    """G=4, lhs f32 [512,256], rhs f32 [4,384,256] NT, both N(0,1); group 1
    empty, 480 rows split over groups 0, 2, 3; rows 480..511 unassigned."""
    sizes = multinomial_group_sizes(seed, 480, 4, empty=(1,))
    lhs = normal((512, 256), 1.0, seed + 1, device)
    rhs = normal((4, 384, 256), 1.0, seed + 2, device)
    return Case("tiny_fp32", lhs, rhs, torch.from_numpy(sizes).to(device),
                out_dtype=torch.float32,
                meta=dict(tokens=None, experts=4))


def moe_forward_bf16(seed: int = 1002, device="cpu", tokens: int = 32768, experts: int = 128,
                     top_k: int = 8, K: int = 1408, N: int = 1408, std: float = 0.02,
                     sizes_seed: Optional[int] = None) -> Case:
    """MoE up-projection forward: lhs bf16 [tokens*top_k, K] N(0,std), rhs
    bf16 [experts, N, K] N(0,std) (NT), router group sizes, bf16 out."""
    sizes = router_group_sizes(sizes_seed if sizes_seed is not None else seed, tokens, experts, top_k)
    M = tokens * top_k
    lhs = normal((M, K), std, seed + 1, device, torch.bfloat16)
    rhs = normal((experts, N, K), std, seed + 2, device, torch.bfloat16)
    return Case("moe_fwd_bf16", lhs, rhs, torch.from_numpy(sizes).to(device),
                meta=dict(tokens=tokens, experts=experts, top_k=top_k))


def moe_dlhs_bf16(seed: int = 1003, device="cpu", tokens: int = 32768, experts: int = 128,
                  top_k: int = 8, K: int = 1408, N: int = 704, dout_std: float = 1e-3,
                  w_std: float = 0.02, sizes_seed: int = 1002) -> Case:
    """Backward dlhs of the down-projection: dout bf16 [tokens*top_k, K]
    N(0,dout_std); the forward weight W bf16 [experts, K, N] N(0,w_std) is
    read in place (transpose_rhs, an NN product); dlhs [M, N] bf16."""
    sizes = router_group_sizes(sizes_seed, tokens, experts, top_k)
    M = tokens * top_k
    lhs = normal((M, K), dout_std, seed + 1, device, torch.bfloat16)
    rhs = normal((experts, K, N), w_std, seed + 2, device, torch.bfloat16)
    return Case("moe_dlhs_bf16", lhs, rhs, torch.from_numpy(sizes).to(device),
                transpose_rhs=True, meta=dict(tokens=tokens, experts=experts, top_k=top_k))


def decode_fp8_weight(seed: int = 1004, device="cpu", tokens: int = 256, experts: int = 128,
                      top_k: int = 8, K: int = 1408, N: int = 1408, forced_empty: int = 51,
                      group_offset: int = 32, num_active: int = 64) -> Case:
    """Decode-sized fp8-weight gmm: lhs bf16 [tokens*top_k, K] N(0,1);
    W N(0,1) quantised per (expert, n, 128-K block) to e4m3 with rhs_scale
    f32 [experts, K/128, 1, N]; rhs_bias bf16 [experts, 1, N] N(0, sqrt(K));
    ``forced_empty`` experts have no rows; groups group_offset ..
    group_offset+num_active-1 are active and rhs / scale / bias are that
    shard."""
    sizes = router_group_sizes(seed, tokens, experts, top_k, forced_empty=forced_empty)
    M = tokens * top_k
    lhs = normal((M, K), 1.0, seed + 1, device, torch.bfloat16)
    q, sc = _quantized_weight(experts, N, K, 1.0, seed + 2, device)
    bias = normal((experts, 1, N), math.sqrt(K), seed + 3, device, torch.bfloat16)
    sl = slice(group_offset, group_offset + num_active)
    return Case("decode_fp8w", lhs, q[sl].contiguous(), torch.from_numpy(sizes).to(device),
                group_offset=group_offset, rhs_scale=sc[sl].contiguous(),
                rhs_bias=bias[sl].contiguous(),
                meta=dict(tokens=tokens, experts=experts, top_k=top_k))


def w8a8_fp8(seed: int = 1005, device="cpu", tokens: int = 32768, experts: int = 128,
             top_k: int = 8, K: int = 1408, N: int = 704, std: float = 0.02,
             sizes_seed: int = 1002) -> Case:
    """W8A8: lhs N(0,std) [tokens*top_k, K] quantised per token per 128-K
    block to e4m3 with lhs_scale f32 [M, K/128]; W N(0,std) [experts, N, K]
    quantised per (expert, n, block) with rhs_scale [experts, K/128, 1, N];
    bf16 out."""
    sizes = router_group_sizes(sizes_seed, tokens, experts, top_k)
    M = tokens * top_k
    x = normal((M, K), std, seed + 1, device)
    lq, ls = quantize_e4m3_blocks(x)
    del x
    q, sc = _quantized_weight(experts, N, K, std, seed + 2, device)
    return Case("w8a8_fp8", lq, q, torch.from_numpy(sizes).to(device),
                rhs_scale=sc, lhs_scale=ls,
                meta=dict(tokens=tokens, experts=experts, top_k=top_k))


@dataclasses.dataclass
class TgmmCase:
    """Inputs of the transposed grouped matmul (weight gradient):
    out[h] = lhs_g^T . rhs_g over the rows of group g = group_offset + h."""
    name: str
    lhs: torch.Tensor               # [M,K]
    rhs: torch.Tensor               # [M,N]
    group_sizes: torch.Tensor       # int32 [G]
    num_active: int
    group_offset: int = 0
    out_dtype: torch.dtype = torch.float32
    meta: Dict = dataclasses.field(default_factory=dict)

    @property
    def M(self):
        return self.lhs.shape[0]

    @property
    def K(self):
        return self.lhs.shape[1]

    @property
    def N(self):
        return self.rhs.shape[1]

    def sizes_list(self):
        return [int(x) for x in self.group_sizes.cpu().tolist()]

    def active_rows(self):
        s = self.sizes_list()
        return sum(s[self.group_offset:self.group_offset + self.num_active])

    def flops(self):
        """2 * (active rows) * K * N."""
        return 2 * self.active_rows() * self.K * self.N

    def algorithmic_bytes(self):
        """Active rows of both operands, every output element (empty groups
        are written as zeros) and the group sizes."""
        r = self.active_rows()
        b = r * self.K * self.lhs.element_size() + r * self.N * self.rhs.element_size()
        b += self.num_active * self.K * self.N * torch.tensor([], dtype=self.out_dtype).element_size()
        return b + self.group_sizes.numel() * 4


def tgmm_bf16(seed: int = 1006, device="cpu", tokens: int = 32768, experts: int = 128,
              top_k: int = 8, K: int = 1408, N: int = 1408, sizes_seed: int = 1002) -> TgmmCase:
    """Weight gradient of the MoE up-projection (the drhs of the forward
    workload): lhs = the forward's activations, bf16 [tokens*top_k, K]
    N(0, 0.02); rhs = the output gradient, bf16 [tokens*top_k, N] N(0, 1e-3)
    (the dlhs workload's dout); the forward's router group sizes; f32 out
    [experts, K, N]."""
    sizes = router_group_sizes(sizes_seed, tokens, experts, top_k)
    M = tokens * top_k
    lhs = normal((M, K), 0.02, seed + 1, device, torch.bfloat16)
    rhs = normal((M, N), 1e-3, seed + 2, device, torch.bfloat16)
    return TgmmCase("tgmm_bf16", lhs, rhs, torch.from_numpy(sizes).to(device), num_active=experts,
                    meta=dict(tokens=tokens, experts=experts, top_k=top_k))


@dataclasses.dataclass
class QuantCase:
    """Input of the per-token activation quantiser: x bf16 [M,K], blocks of
    ``block`` elements along each row."""
    name: str
    x: torch.Tensor
    block: int = 128
    meta: Dict = dataclasses.field(default_factory=dict)

    @property
    def M(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    def active_rows(self):
        return self.M

    def flops(self):
        return 0

    def algorithmic_bytes(self):
        """x read once (2 bytes an element), the codes written once (1 byte)
        and one f32 scale per block."""
        return self.M * self.K * 3 + self.M * (self.K // self.block) * 4

    def to(self, device):
        return dataclasses.replace(self, x=self.x.to(device))


def quant_fp8_act(seed: int = 1002, device="cpu", tokens: int = 32768, top_k: int = 8, K: int = 1408,
                  std: float = 0.02) -> QuantCase:
    """The forward workload's activations, bf16 [tokens*top_k, K] N(0,std)
    (the same draw as moe_forward_bf16's lhs), to be quantised per token per
    128-element block for the W8A8 product."""
    x = normal((tokens * top_k, K), std, seed + 1, device, torch.bfloat16)
    return QuantCase("quant_fp8", x, meta=dict(tokens=tokens, top_k=top_k))


QUANT_FULL = {
    "quant_fp8": lambda device="cpu": quant_fp8_act(device=device),
}


TGMM_FULL = {
    "tgmm_bf16": lambda device="cpu": tgmm_bf16(device=device),
}


FULL = {
    "tiny_fp32": lambda device="cpu": tiny_fp32(device=device),
    "moe_fwd_bf16": lambda device="cpu": moe_forward_bf16(device=device),
    "moe_dlhs_bf16": lambda device="cpu": moe_dlhs_bf16(device=device),
    "decode_fp8w": lambda device="cpu": decode_fp8_weight(device=device),
    "w8a8_fp8": lambda device="cpu": w8a8_fp8(device=device),
}

# Reduced sizes of the same recipes: the oracle finishes them in seconds, yet
# they span several tiles in M, N and K, ragged group boundaries, empty
# groups and an N tail.
SMALL = {
    "tiny_fp32": lambda device="cpu": tiny_fp32(device=device),
    "moe_fwd_bf16": lambda device="cpu": moe_forward_bf16(
        device=device, tokens=384, experts=16, K=512, N=576, sizes_seed=77),
    "moe_dlhs_bf16": lambda device="cpu": moe_dlhs_bf16(
        device=device, tokens=384, experts=16, K=576, N=320, sizes_seed=77),
    "decode_fp8w": lambda device="cpu": decode_fp8_weight(
        device=device, tokens=64, experts=32, K=768, N=640, forced_empty=12,
        group_offset=8, num_active=16),
    "w8a8_fp8": lambda device="cpu": w8a8_fp8(
        device=device, tokens=384, experts=16, K=512, N=320, sizes_seed=77),
}
