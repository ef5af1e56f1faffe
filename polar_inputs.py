"""Seeded synthetic inputs for the Polar Attention workloads.

This module only draws random numbers and plants structure; it holds none of the
method's arithmetic.  Both the GPU tests/benchmark and the CPU oracle consume what it
returns, so the two sides always see identical tensors.

Recipe: q, k, v are drawn, in that order, from one seeded CPU torch.Generator as fp32
N(0,1) and rounded to bf16 (round to nearest even) unless the workload is fp32.
Planted structure comes from a second generator seeded with seed + 1 and is applied
after rounding (a factor 4 is exact in bf16).  The decode workload is too large to draw
on the host in reasonable time, so it is drawn on the device with a seeded device
generator, one batch element at a time; tests copy the slices they check back to the
host for the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

# Planted-match strength: a planted key is this multiple of its target query.
PLANT_SCALE = 4.0
# Match-group multiplicities of the 16K workload.
GROUP_SIZES = (1, 4, 16, 64)


@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    B: int
    H: int
    Hkv: int
    Tq: int
    Tk: int
    d: int
    causal: bool
    seed: int
    plant: str | None = None          # None | "needle" | "groups"
    tau_step: float = 0.0             # tau_h = tau_step * h
    floor_on: bool = True             # beta_h = 0 when on, floor off when False
    decode: bool = False
    description: str = ""
    extra: dict = field(default_factory=dict)

    def len_temp(self):
        return [self.tau_step * h for h in range(self.H)]

    def null_bias(self):
        return [0.0] * self.H if self.floor_on else None

    def count_scale(self):
        return [1.0] * self.H

    def pairs(self) -> int:
        """(query, key) pairs whose score the operator must compute."""
        if self.causal and not self.decode:
            off = self.Tk - self.Tq          # rows are aligned to the end of the keys (Tq <= Tk)
            return self.B * self.H * (self.Tq * (self.Tq + 1) // 2 + off * self.Tq)
        return self.B * self.H * self.Tq * self.Tk


WORKLOADS = {
    "fp32_b1_h2_t256_d64": Workload(
        "fp32_b1_h2_t256_d64", torch.float32, 1, 2, 2, 256, 256, 64, True, 1001,
        description="Polar Attention forward, fp32, B=1 H=2 T=256 d=64, causal, i.i.d. N(0,1)"),
    "bf16_b4_h8_t4096_d64_needle": Workload(
        "bf16_b4_h8_t4096_d64_needle", torch.bfloat16, 4, 8, 8, 4096, 4096, 64, True, 1002, plant="needle",
        description="Polar Attention forward, bf16, B=4 H=8 T=4096 d=64, causal, one planted needle per head"),
    "bf16_b1_h16_t16384_d128_groups": Workload(
        "bf16_b1_h16_t16384_d128_groups", torch.bfloat16, 1, 16, 16, 16384, 16384, 128, True, 1003,
        plant="groups",
        description="Polar Attention forward, bf16, B=1 H=16 T=16384 d=128, causal, match groups {1,4,16,64}"),
    "bf16_b1_h16_t65536_d64_lentemp": Workload(
        "bf16_b1_h16_t65536_d64_lentemp", torch.bfloat16, 1, 16, 16, 65536, 65536, 64, True, 1004,
        tau_step=0.02,
        description="Polar Attention forward, bf16, B=1 H=16 T=65536 d=64, causal, tau_h = 0.02 h"),
    "bf16_decode_b64_h8_tk65536_d128": Workload(
        "bf16_decode_b64_h8_tk65536_d128", torch.bfloat16, 64, 8, 8, 1, 65536, 128, True, 1005, decode=True,
        description="Polar Attention split-KV decode, bf16, batch 64, H=8, d=128, 65536-token KV cache"),
    "bf16_paged_decode_b64_h32_kv8_tk65536_d128": Workload(
        "bf16_paged_decode_b64_h32_kv8_tk65536_d128", torch.bfloat16, 64, 32, 8, 1, 65536, 128, False, 1006,
        decode=True, extra={"block_size": 16},
        description="Polar Attention grouped split-KV decode over a paged cache, bf16, batch 64, 32 query heads "
                    "over 8 KV heads, d=128, 65536 keys per sequence in shuffled 16-row blocks"),
    "bf16_bwd_b1_h16_kv4_t16384_d128": Workload(
        "bf16_bwd_b1_h16_kv4_t16384_d128", torch.bfloat16, 1, 16, 4, 16384, 16384, 128, True, 1007,
        tau_step=0.01, extra={"grad_seed": 1107},
        description="Polar Attention backward, bf16 inputs, B=1, 16 query heads over 4 KV heads, T=16384, d=128, "
                    "causal, tau_h = 0.01 h, N(0,1) upstream gradients of all four channels"),
}


def _plant_needles(q, k, g2, meta):
    B, H, T, _ = q.shape
    needles = []
    for b in range(B):
        for h in range(H):
            i_star = int(torch.randint(1, T, (1,), generator=g2))
            j_star = int(torch.randint(0, i_star, (1,), generator=g2))
            k[b, h, j_star] = PLANT_SCALE * q[b, h, i_star]
            needles.append((b, h, i_star, j_star))
    meta["needles"] = needles


def _plant_groups(q, k, g2, meta):
    B, H, T, _ = q.shape
    groups = []
    for b in range(B):
        for h in range(H):
            targets = (T // 2 + torch.randperm(T - T // 2, generator=g2)[:len(GROUP_SIZES)]).tolist()
            used = set()
            for c, i_c in zip(GROUP_SIZES, targets):
                order = torch.randperm(i_c, generator=g2).tolist()
                pos = []
                for j in order:
                    if j not in used:
                        pos.append(j)
                        used.add(j)
                        if len(pos) == c:
                            break
                assert len(pos) == c
                for j in pos:
                    k[b, h, j] = PLANT_SCALE * q[b, h, i_c]
                groups.append((b, h, c, i_c, sorted(pos)))
    meta["groups"] = groups


def random_qkv(B, H, Hkv, Tq, Tk, d, dtype=torch.bfloat16, seed=0, plant=None):
    """q [B,H,Tq,d], k and v [B,Hkv,Tk,d] on the host, plus planting metadata."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Tq, d, generator=g, dtype=torch.float32).to(dtype)
    k = torch.randn(B, Hkv, Tk, d, generator=g, dtype=torch.float32).to(dtype)
    v = torch.randn(B, Hkv, Tk, d, generator=g, dtype=torch.float32).to(dtype)
    meta = {}
    if plant is not None:
        assert H == Hkv and Tq == Tk, "planted structure assumes self-attention with one kv head per head"
        g2 = torch.Generator().manual_seed(seed + 1)
        if plant == "needle":
            _plant_needles(q, k, g2, meta)
        elif plant == "groups":
            _plant_groups(q, k, g2, meta)
        else:
            raise ValueError(plant)
    return q, k, v, meta


def random_grads(B, H, Tq, d, seed, names=("direction", "n_eff", "confidence", "count")):
    """Upstream gradients of the four output channels, i.i.d. N(0, 1) fp32 on the host
    (direction [B,H,Tq,d], the others [B,H,Tq]); only the channels in `names`."""
    g = torch.Generator().manual_seed(seed)
    shapes = {"direction": (B, H, Tq, d), "n_eff": (B, H, Tq), "confidence": (B, H, Tq), "count": (B, H, Tq)}
    out = {}
    for name in ("direction", "n_eff", "confidence", "count"):
        x = torch.randn(shapes[name], generator=g, dtype=torch.float32)  # drawn for every name: stable streams
        if name in names:
            out[name] = x
    return out


def workload_inputs(w: Workload, device="cpu"):
    """Inputs of a named workload.  Prefill workloads are drawn on the host and moved
    to `device`; the decode workload is drawn directly on `device`."""
    if w.decode:
        return decode_inputs(w, device)
    q, k, v, meta = random_qkv(w.B, w.H, w.Hkv, w.Tq, w.Tk, w.d, w.dtype, w.seed, w.plant)
    if device != "cpu":
        q, k, v = q.to(device), k.to(device), v.to(device)
    return q, k, v, meta


def decode_inputs(w: Workload, device):
    """Decode workload: q [B,H,1,d], KV cache [B,Hkv,Tk,d], drawn per batch element from
    a device generator seeded with seed * 1000 + b (q from seed * 1000 - 1)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed * 1000 - 1)
    q = torch.randn(w.B, w.H, w.Tq, w.d, generator=g, device=dev, dtype=torch.float32).to(w.dtype)
    k = torch.empty(w.B, w.Hkv, w.Tk, w.d, device=dev, dtype=w.dtype)
    v = torch.empty_like(k)
    for b in range(w.B):
        g.manual_seed(w.seed * 1000 + b)
        k[b] = torch.randn(w.Hkv, w.Tk, w.d, generator=g, device=dev, dtype=torch.float32).to(w.dtype)
        v[b] = torch.randn(w.Hkv, w.Tk, w.d, generator=g, device=dev, dtype=torch.float32).to(w.dtype)
    return q, k, v, {}


def paged_decode_inputs(w: Workload, device):
    """Paged decode workload: q [B,H,1,d]; pools [NB, block_size, Hkv, d] holding every
    sequence's Tk keys in blocks placed at a random permutation of the pool (block table
    [B, Tk / block_size] int32, from a CPU generator seeded with seed + 1); seq_lens [B]
    = Tk.  The keys of sequence b are drawn like the contiguous decode workload's, from a
    device generator seeded with seed * 1000 + b (q from seed * 1000 - 1)."""
    dev = torch.device(device)
    bs = w.extra["block_size"]
    mb = w.Tk // bs
    nb = w.B * mb
    table = torch.randperm(nb, generator=torch.Generator().manual_seed(w.seed + 1)).view(w.B, mb)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed * 1000 - 1)
    q = torch.randn(w.B, w.H, w.Tq, w.d, generator=g, device=dev, dtype=torch.float32).to(w.dtype)
    k_pool = torch.empty(nb, bs, w.Hkv, w.d, device=dev, dtype=w.dtype)
    v_pool = torch.empty_like(k_pool)
    rows = table.to(dev)
    for b in range(w.B):
        g.manual_seed(w.seed * 1000 + b)
        for pool in (k_pool, v_pool):
            x = torch.randn(w.Hkv, w.Tk, w.d, generator=g, device=dev, dtype=torch.float32).to(w.dtype)
            pool[rows[b]] = x.view(w.Hkv, mb, bs, w.d).permute(1, 2, 0, 3)
    lens = torch.full((w.B,), w.Tk, dtype=torch.int32, device=dev)
    return q, k_pool, v_pool, rows.to(torch.int32), lens


# Rows whose weights sit near bf16 rounding boundaries, for the n_eff precision tests:
# per head, (strong key value, weak key value) along dimension 0.  With q = e_0 every
# row's scores are exactly the key values; key 0 scores 0, key 64 scores the strong value
# and every other key the weak value, so row i sees one key of weight 1, one strong key
# and i - 1 identical weak keys (the weights relative to the row's maximum in the first
# 64 keys).  The pairs were picked so that the strong key's and the weak keys' weights,
# formed in fp32, round to bf16 in opposite directions by nearly half an ulp.
ROUNDING_PAIRS = {
    64: ((50.0, -5.03125), (39.5, -10.8125), (50.0, -10.875), (50.0, -4.25)),
    128: ((56.5, -15.125), (56.5, -7.625), (48.5, -15.375), (24.5, -38.0)),
}


def rounding_adversary_qkv(T, d, seed=0, pairs=None):
    """q, k, v (bf16, [1, H, T, d]) with one (strong, weak) key-value pair per head as
    ROUNDING_PAIRS describes; v is N(0,1) from `seed`, and the key dimensions other than
    0 are N(0,1) too (q is zero there, so they do not change any score)."""
    pairs = ROUNDING_PAIRS[d] if pairs is None else pairs
    H = len(pairs)
    g = torch.Generator().manual_seed(seed)
    q = torch.zeros(1, H, T, d)
    q[..., 0] = 1.0
    k = torch.randn(1, H, T, d, generator=g)
    v = torch.randn(1, H, T, d, generator=g)
    for h, (strong, weak) in enumerate(pairs):
        k[0, h, :, 0] = weak
        k[0, h, 0, 0] = 0.0
        if T > 64:
            k[0, h, 64, 0] = strong
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
