"""GPU parity of the grouped split-KV decode over contiguous and paged caches.

The oracle sees each sequence's keys as one contiguous array (its first seq_len rows);
the GPU reads them from a pool of blocks in shuffled order through the block table.
Unused pool slots hold random values, so a wrong block or row index shows up as a
parity failure.  Grouped means several query heads share one KV head; the kernel reads
every K and V row once per group (up to 8 query heads per workgroup).
"""
import math

import numpy as np
import pytest
import torch

import long_context_attention_polar_amd as pa
import polar_inputs as pin
from oracle import merge_reference, polar_attention
from tests.parity import assert_parity, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def make_paged(k, v, block_size, seed, spare=3):
    """Scatter caches k, v [B, Hkv, Tk, d] into pools [NB, block_size, Hkv, d] with the
    logical blocks of every sequence at random pool blocks; returns (k_pool, v_pool,
    block_table [B, ceil(Tk / block_size)] int32)."""
    B, Hkv, Tk, d = k.shape
    mb = math.ceil(Tk / block_size)
    nb = B * mb + spare
    g = torch.Generator().manual_seed(seed)
    table = torch.randperm(nb, generator=g)[:B * mb].view(B, mb)
    k_pool = torch.randn(nb, block_size, Hkv, d, generator=g).to(k.dtype)
    v_pool = torch.randn(nb, block_size, Hkv, d, generator=g).to(v.dtype)
    for b in range(B):
        for j in range(mb):
            lo, hi = j * block_size, min(Tk, (j + 1) * block_size)
            k_pool[table[b, j], :hi - lo] = k[b, :, lo:hi].permute(1, 0, 2)
            v_pool[table[b, j], :hi - lo] = v[b, :, lo:hi].permute(1, 0, 2)
    return k_pool, v_pool, table.to(torch.int32)


def oracle_per_sequence(q, k, v, lens, tau=None, beta=None, kappa=None):
    """Oracle outputs [B, H, 1, ...] where sequence b sees its first lens[b] keys."""
    B, H = q.shape[0], q.shape[1]
    parts = []
    for b in range(B):
        L = int(lens[b])
        parts.append(polar_attention(to_np(q[b:b + 1]), to_np(k[b:b + 1, :, :L]), to_np(v[b:b + 1, :, :L]),
                                     causal=False, len_temp=tau, null_bias=beta, count_scale=kappa))
    return {key: np.concatenate([p[key] for p in parts], axis=0) for key in parts[0]}


def paged_case(B, H, Hkv, lens, d, block_size, seed, splits_list, tau=None, beta=None, kappa=None):
    Tk = max(lens)
    q, k, v, _ = pin.random_qkv(B, H, Hkv, 1, Tk, d, torch.bfloat16, seed)
    kp, vp, table = make_paged(k, v, block_size, seed + 1)
    ref = oracle_per_sequence(q, k, v, lens, tau, beta, kappa)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    args = (q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), lens_t.to(DEV))
    outs = []
    for s in splits_list:
        out = pa.decode_paged(*args, seq_k=Tk, num_splits=s, len_temp=tau, null_bias=beta, count_scale=kappa,
                              stats=True)
        torch.cuda.synchronize()
        label = f"paged B={B} H={H} Hkv={Hkv} d={d} bs={block_size} S={s}"
        assert_parity(out, ref, "bf16", label=label)
        # per sequence, the oracle's merge of the GPU partials with n = that sequence's length
        parts = to_np(out["partials"])
        for b in range(B):
            merged = merge_reference(parts[b:b + 1], lens[b], len_temp=tau, null_bias=beta, count_scale=kappa)
            one = {key: (val[b:b + 1] if val is not None else None) for key, val in out.items()
                   if key in ("direction", "n_eff", "confidence", "count", "stats")}
            assert_parity(one, merged, "bf16", label=label + f" oracle merge b={b}")
        outs.append(out)
    return outs


@pytest.mark.parametrize("d", [64, 128])
def test_paged_gqa_against_oracle(d):
    paged_case(3, 8, 2, [1, 333, 700], d, 16, seed=200 + d, splits_list=[1, 3, 0],
               tau=[0.0, 0.1, 0.2, 0.05, 0.0, 0.3, 0.1, 0.0], beta=[0.0, -1.0, 2.0, 0.0, 1.0, 0.0, 0.0, -2.0],
               kappa=[1.0, 2.0, 1.0, 4.0, 1.0, 1.0, 3.0, 1.0])


@pytest.mark.parametrize("group,block_size", [(1, 1), (2, 8), (3, 64), (4, 16), (6, 32), (8, 16), (16, 128)])
def test_paged_group_sizes_and_block_sizes(group, block_size):
    """Group chunks of 8, 4, 2 and 1 heads, and block sizes from one row to 128 rows."""
    paged_case(2, 2 * group, 2, [257, 130], 128, block_size, seed=300 + group, splits_list=[2, 0],
               beta=[0.0] * (2 * group))


@pytest.mark.parametrize("Tk", [1000, 5500])
def test_paged_equals_contiguous_bitwise(Tk):
    """The same grouped kernel over a shuffled pool and over the contiguous cache: only
    row addresses differ, so the partials and the outputs are bitwise equal.  At 5500
    keys the automatic split count of the paged call is above one (a split keeps at
    least 2048 keys), so the automatic choice is exercised with several splits."""
    B, H, Hkv, d = 2, 8, 2, 128
    q, k, v, _ = pin.random_qkv(B, H, Hkv, 1, Tk, d, torch.bfloat16, 77 + Tk)
    kp, vp, table = make_paged(k, v, 16, 78)
    lens = torch.full((B,), Tk, dtype=torch.int32)
    ref = oracle_per_sequence(q, k, v, [Tk] * B, beta=[0.0] * H)
    for s in (1, 5, 0):
        # 0: the paged call's automatic split count, which the contiguous call then uses
        pag = pa.decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), lens.to(DEV), seq_k=Tk,
                              num_splits=s, null_bias=[0.0] * H, stats=True)
        cont = pa.decode(q.to(DEV), k.to(DEV), v.to(DEV), num_splits=pag["splits"], null_bias=[0.0] * H,
                         stats=True)
        torch.cuda.synchronize()
        assert cont["splits"] == pag["splits"] and (s == 0 or pag["splits"] == s)
        if s == 0 and Tk > 4096:
            assert pag["splits"] > 1, pag["splits"]
        assert torch.equal(cont["partials"], pag["partials"]), s
        for key in ("direction", "n_eff", "confidence", "count", "stats"):
            assert torch.equal(cont[key], pag[key]), (s, key)
        assert_parity(pag, ref, "bf16", label=f"paged Tk={Tk} S={pag['splits']}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H", [4, 8, 16])
def test_grouped_matches_per_head_reads(d, H):
    """GQA (2, 4 or 8 query heads per KV head) against the same caches repeated for every
    query head (plain multi-head layout): equal up to fp32 summation order.  At head_dim
    128 the grouped kernel splits the heads over the lanes of a key for the dot's sum."""
    B, Hkv, Tk = 2, 2, 900
    q, k, v, _ = pin.random_qkv(B, H, Hkv, 1, Tk, d, torch.bfloat16, 91)
    rep_k = k.repeat_interleave(H // Hkv, dim=1).contiguous()
    rep_v = v.repeat_interleave(H // Hkv, dim=1).contiguous()
    lens = [Tk, 450]
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kp, vp, table = make_paged(k, v, 32, 92)
    kr, vr, table_r = make_paged(rep_k, rep_v, 32, 93)
    g = pa.decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), lens_t, seq_k=Tk, num_splits=4,
                        stats=True)
    u = pa.decode_paged(q.to(DEV), kr.to(DEV), vr.to(DEV), table_r.to(DEV), lens_t, seq_k=Tk, num_splits=4,
                        stats=True)
    torch.cuda.synchronize()
    for key in ("direction", "n_eff", "stats"):
        diff = (g[key] - u[key]).abs().max().item()
        assert diff <= 1e-4 * max(1.0, u[key].abs().max().item()), (key, diff)
    assert_parity(g, oracle_per_sequence(q, k, v, lens), "bf16", label="grouped")


def test_paged_empty_sequence_and_bad_table_entries():
    """A sequence with no keys gets zeros; a table entry outside the pool is skipped
    (never read): that sequence's outputs stay finite and the others are unaffected."""
    B, H, Hkv, d = 3, 4, 2, 128
    lens = [0, 40, 70]
    q, k, v, _ = pin.random_qkv(B, H, Hkv, 1, 70, d, torch.bfloat16, 121)
    kp, vp, table = make_paged(k, v, 16, 122)
    table[1, 1] = -1                   # keys 16..31 of sequence 1 are skipped
    table[1, 2] = kp.shape[0]          # and keys 32..39
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = pa.decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), lens_t, seq_k=70, stats=True)
    torch.cuda.synchronize()
    assert torch.all(out["direction"][0] == 0) and torch.all(out["n_eff"][0] == 0)
    assert torch.all(out["confidence"][0] == 0) and torch.all(out["count"][0] == 0)
    assert torch.isfinite(out["direction"][1]).all() and torch.isfinite(out["n_eff"][1]).all()
    ref = oracle_per_sequence(q[2:], k[2:], v[2:], [70])
    third = {key: (val[2:] if val is not None else None) for key, val in out.items()
             if key in ("direction", "n_eff", "confidence", "count", "stats")}
    assert_parity(third, ref, "bf16", label="unaffected sequence")


def test_paged_binding_rejects_bad_tensors():
    q = torch.zeros(1, 2, 1, 64, dtype=torch.bfloat16, device=DEV)
    kp = torch.zeros(4, 16, 2, 64, dtype=torch.bfloat16, device=DEV)
    table = torch.zeros(1, 4, dtype=torch.int64, device=DEV)
    lens = torch.ones(1, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        pa.decode_paged(q, kp, kp.clone(), table, lens)
    with pytest.raises(ValueError):  # 3 rows per block is not a power of two
        pa.decode_paged(q, kp[:, :3].contiguous(), kp[:, :3].contiguous(), table.to(torch.int32), lens)


def test_workload_paged_decode_64k():
    """The benchmark's paged GQA decode at full size, every (sequence, query head) row
    against the oracle: for each (sequence, KV head) the oracle reads that sequence's keys
    back out of the pool in logical order and computes all query heads of the group."""
    w = pin.WORKLOADS["bf16_paged_decode_b64_h32_kv8_tk65536_d128"]
    print("[parity] paged decode workload", flush=True)
    q, kp, vp, table, lens = pin.paged_decode_inputs(w, DEV)
    out = pa.decode_paged(q, kp, vp, table, lens, seq_k=w.Tk, len_temp=w.len_temp(), null_bias=w.null_bias(),
                          count_scale=w.count_scale(), stats=True)
    torch.cuda.synchronize()
    assert out["splits"] > 1
    group = w.H // w.Hkv
    worst = {}
    for b in range(w.B):
        rows = table[b].long()
        for hk in range(w.Hkv):
            heads = slice(hk * group, (hk + 1) * group)
            kb = kp[rows, :, hk].reshape(1, 1, w.Tk, w.d)
            vb = vp[rows, :, hk].reshape(1, 1, w.Tk, w.d)
            ref = polar_attention(to_np(q[b:b + 1, heads]), to_np(kb), to_np(vb), causal=False,
                                  len_temp=w.len_temp()[heads], null_bias=w.null_bias()[heads],
                                  count_scale=w.count_scale()[heads])
            sub = {key: (t[b:b + 1, heads] if torch.is_tensor(t) else t) for key, t in out.items()
                   if key not in ("partials", "splits")}
            e = assert_parity(sub, ref, "bf16", label=f"paged decode b={b} hk={hk}")
            worst = {n: max(worst.get(n, 0.0), x) for n, x in e.items()}
    print(f"[parity] paged decode max errors over all {w.B * w.H} rows {worst}", flush=True)
    del kp, vp
    torch.cuda.empty_cache()
