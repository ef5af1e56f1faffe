"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

Every call below is rejected by the library's argument checks, which run before the
first HIP call, so nothing touches a device.  Pointers are fake but aligned addresses.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import long_context_attention_polar_amd as pa
from long_context_attention_polar_amd import build as pbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "polar_attn.h")


@pytest.fixture(scope="module")
def lib():
    # POLAR_TEST_LIB: another build of the library to run these checks against (the
    # host-sanitizer build of tests/test_host_sanitizers.py)
    path = os.environ.get("POLAR_TEST_LIB")
    if path:
        return pa.load_library(path)
    if not os.path.exists(pa.LIB_PATH):
        pbuild.build()
    return pa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(polar_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("polar_attn_fwd", "polar_attn_decode", "polar_attn_merge", "polar_attn_decode_workspace_bytes",
                     "polar_attn_decode_num_splits", "polar_status_string", "polar_abi_version"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        getattr(lib, n)


def test_abi_version_and_status_strings(lib):
    version = int(re.search(r"#define POLAR_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert pa.abi_version() == version
    for s in range(9):
        assert pa.status_string(s) and pa.status_string(s) != "unknown status"
    assert pa.status_string(99) == "unknown status"


def test_ctypes_struct_layout_matches_header(tmp_path):
    """The binding's ctypes structures have the header's offsets and sizes (checked by
    compiling the header with the host C compiler)."""
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "polar_attn.h"\n'
        "#define F(T, m) printf(#T \" \" #m \" %zu\\n\", offsetof(T, m));\n"
        "int main(void) {\n"
        "F(polar_problem, batch) F(polar_problem, heads) F(polar_problem, kv_heads) F(polar_problem, seq_q)\n"
        "F(polar_problem, seq_k) F(polar_problem, head_dim) F(polar_problem, causal) F(polar_problem, dtype)\n"
        "F(polar_problem, softmax_scale) F(polar_problem, len_temp) F(polar_problem, null_bias)\n"
        "F(polar_problem, count_scale) F(polar_problem, variant)\n"
        "F(polar_variant, temperature) F(polar_variant, train_len) F(polar_variant, floor_level)\n"
        "F(polar_variant, key_floor) F(polar_variant, saturation) F(polar_variant, window)\n"
        "F(polar_outputs, direction) F(polar_outputs, n_eff) F(polar_outputs, confidence) F(polar_outputs, count)\n"
        "F(polar_outputs, stats)\n"
        "F(polar_paged_kv, k_pool) F(polar_paged_kv, v_pool) F(polar_paged_kv, block_table)\n"
        "F(polar_paged_kv, seq_lens) F(polar_paged_kv, num_blocks) F(polar_paged_kv, block_size)\n"
        "F(polar_paged_kv, max_blocks)\n"
        "F(polar_grads, d_direction) F(polar_grads, d_n_eff) F(polar_grads, d_confidence) F(polar_grads, d_count)\n"
        'printf("sizeof polar_problem %zu\\nsizeof polar_outputs %zu\\n", sizeof(polar_problem), sizeof(polar_outputs));\n'
        'printf("sizeof polar_paged_kv %zu\\n", sizeof(polar_paged_kv));\n'
        'printf("sizeof polar_grads %zu\\n", sizeof(polar_grads));\n'
        'printf("sizeof polar_variant %zu\\n", sizeof(polar_variant));\n'
        "return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    classes = {"polar_problem": pa.PolarProblem, "polar_outputs": pa.PolarOutputs, "polar_paged_kv": pa.PolarPagedKV,
               "polar_grads": pa.PolarGrads, "polar_variant": pa.PolarVariant}
    for line in filter(None, lines):
        a, b, c = line.split()
        if a == "sizeof":
            assert ctypes.sizeof(classes[b]) == int(c), line
        else:
            assert getattr(classes[a], b).offset == int(c), line


# ---------------------------------------------------------------- argument checks (no launch)

FAKE = 1 << 40  # aligned, never dereferenced: every call below fails validation first


def fake(n=0):
    return ctypes.c_void_p(FAKE + n * (1 << 34))


def good_problem(**kw):
    base = dict(batch=1, heads=2, kv_heads=2, seq_q=64, seq_k=64, head_dim=64, causal=True, dtype=pa.POLAR_BF16)
    base.update(kw)
    return pa.Problem(**base)


def outputs(direction=None, n_eff=None, confidence=None, count=None, stats=None):
    d = fake(10) if direction is None else direction
    n = fake(11) if n_eff is None else n_eff
    return pa.PolarOutputs(d, n, confidence, count, stats)


def call_fwd(lib, prob, q=None, k=None, v=None, out=None):
    pr, keep = prob.to_c()
    o = outputs() if out is None else out
    return lib.polar_attn_fwd(ctypes.byref(pr), fake(1) if q is None else q, fake(2) if k is None else k,
                              fake(3) if v is None else v, ctypes.byref(o), None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), 2), (dict(seq_q=-1), 2), (dict(heads=0), 2), (dict(kv_heads=0), 2), (dict(seq_k=0), 2),
    (dict(heads=3, kv_heads=2), 2), (dict(seq_q=65, seq_k=64), 2), (dict(head_dim=96), 3), (dict(head_dim=256), 3),
    (dict(dtype=7), 3), (dict(softmax_scale=float("nan")), 4), (dict(softmax_scale=float("inf")), 4),
    (dict(len_temp=[0.0, float("nan")]), 4), (dict(len_temp=[0.0, -1.0]), 4), (dict(count_scale=[1.0, 0.0]), 4),
    (dict(count_scale=[1.0, -2.0]), 4), (dict(null_bias=[0.0, float("inf")]), 4),
    (dict(heads=256, kv_heads=256, len_temp=[0.0] * 256), 3),
])
def test_fwd_rejects_bad_problem(lib, kw, status):
    assert call_fwd(lib, good_problem(**kw)) == status


def test_fwd_rejects_bad_pointers(lib):
    prob = good_problem()
    assert call_fwd(lib, prob, q=ctypes.c_void_p(0)) == 1
    assert call_fwd(lib, prob, v=ctypes.c_void_p(0)) == 1
    assert call_fwd(lib, prob, out=outputs(direction=ctypes.c_void_p(0))) == 1
    pr, keep = prob.to_c()
    assert lib.polar_attn_fwd(ctypes.byref(pr), fake(1), fake(2), fake(3), None, None) == 1
    assert lib.polar_attn_fwd(None, fake(1), fake(2), fake(3), ctypes.byref(outputs()), None) == 1
    assert call_fwd(lib, prob, q=ctypes.c_void_p(FAKE + 8)) == 5
    assert call_fwd(lib, prob, out=outputs(direction=ctypes.c_void_p(FAKE + (1 << 36) + 4))) == 5
    assert call_fwd(lib, prob, out=outputs(n_eff=ctypes.c_void_p(FAKE + (1 << 36) + 2))) == 5
    # an output overlapping an input, and two overlapping outputs
    assert call_fwd(lib, prob, out=outputs(direction=fake(1))) == 7
    assert call_fwd(lib, prob, out=outputs(n_eff=ctypes.c_void_p(FAKE + 2 * (1 << 34) + 64))) == 7
    assert call_fwd(lib, prob, out=outputs(count=fake(11))) == 7


def test_bwd_saved_validation(lib):
    """polar_attn_bwd_saved: bf16 only; its workspace is polar_attn_bwd's without the
    forward statistics; `saved` is a required, 16-byte aligned input that no output may
    overlap (unless there are no query rows)."""
    prob = good_problem(batch=2, heads=4, kv_heads=2, seq_q=48, seq_k=64, head_dim=128)
    pr, keep = prob.to_c()
    rows = 2 * 4 * 48
    up = lambda x: (x + 255) // 256 * 256
    full = lib.polar_attn_bwd_workspace_bytes(ctypes.byref(pr))
    ws = lib.polar_attn_bwd_saved_workspace_bytes(ctypes.byref(pr))
    assert ws == full - up(rows * 131 * 4)
    pr32, keep32 = good_problem(dtype=pa.POLAR_F32).to_c()
    assert lib.polar_attn_bwd_saved_workspace_bytes(ctypes.byref(pr32)) == 0
    bad, keep2 = good_problem(head_dim=96).to_c()
    assert lib.polar_attn_bwd_saved_workspace_bytes(ctypes.byref(bad)) == 0
    g = pa.PolarGrads(fake(20), fake(21), None, fake(22))

    def run(saved=8, q=1, dq=4, dk=5, work=7, nbytes=ws, problem=pr):
        arg = lambda x: fake(x) if isinstance(x, int) else x
        return lib.polar_attn_bwd_saved(ctypes.byref(problem), arg(q), fake(2), fake(3), arg(saved), ctypes.byref(g),
                                        arg(dq), arg(dk), fake(6), arg(work), nbytes, None)

    assert run(problem=pr32, nbytes=1 << 30) == 3
    assert run(saved=None) == 1
    assert run(saved=ctypes.c_void_p(FAKE + 8 * (1 << 34) + 8)) == 5
    assert run(nbytes=ws - 1) == 6
    assert run(dq=8) == 7                    # dq over saved
    assert run(work=8) == 7                  # workspace over saved
    # no query rows: saved, q, dq and the workspace may be NULL
    rows0, keep5 = good_problem(seq_q=0, head_dim=128).to_c()
    assert lib.polar_attn_bwd_saved_workspace_bytes(ctypes.byref(rows0)) == 0
    assert run(problem=rows0, saved=None, q=None, dq=None, work=None, nbytes=0, dk=None) == 1   # dk is required


def test_bf16_head_size_limit(lib):
    """bf16 kernels address one head's rows through 32-bit buffer loads: seq * head_dim * 2
    bytes plus 64 KiB must fit; the fp32 kernels have no such limit.  Calls that pass the
    check are stopped by an overlap of outputs, before any launch."""
    overlap = outputs(count=fake(11))
    for d, limit in ((128, 16_776_959), (64, 33_553_919)):
        assert call_fwd(lib, good_problem(seq_k=limit + 1, head_dim=d)) == 3
        assert call_fwd(lib, good_problem(seq_k=limit, head_dim=d), out=overlap) == 7
        assert call_fwd(lib, good_problem(seq_k=limit + 1, head_dim=d, dtype=pa.POLAR_F32), out=overlap) == 7
    pr, keep = good_problem(seq_k=16_776_960, head_dim=128).to_c()
    assert lib.polar_attn_fwd_partial(ctypes.byref(pr), fake(1), fake(2), fake(3), 0, fake(12), 1, 0, None) == 3
    # backward: the limit holds for the queries too
    g = pa.PolarGrads(fake(20), fake(21), None, fake(22))
    for kw in (dict(seq_q=64, seq_k=16_776_960), dict(seq_q=16_776_960, seq_k=64, causal=False)):
        pr, keep = good_problem(head_dim=128, **kw).to_c()
        assert lib.polar_attn_bwd(ctypes.byref(pr), fake(1), fake(2), fake(3), ctypes.byref(g), fake(4), fake(5),
                                  fake(6), fake(7), 1 << 30, None) == 3


def test_negative_tau_within_range_is_accepted_by_validation(lib):
    """1 + tau ln(seq_k) > 0 is the condition; tau = -0.1 at seq_k = 64 passes the check
    (the call is then stopped by an overlap of outputs, before any launch)."""
    prob = good_problem(len_temp=[-0.1, -0.2])
    assert call_fwd(lib, prob, out=outputs(count=fake(11))) == 7


def test_decode_and_merge_validation(lib):
    prob = good_problem(seq_q=1, seq_k=1000, causal=True, head_dim=128)
    pr, keep = prob.to_c()
    assert lib.polar_attn_decode_num_splits(ctypes.byref(pr), 0) >= 1
    assert lib.polar_attn_decode_num_splits(ctypes.byref(pr), 7) == 7
    assert lib.polar_attn_decode_num_splits(ctypes.byref(pr), 1001) == 0
    assert lib.polar_attn_decode_workspace_bytes(ctypes.byref(pr), 5) == 1 * 2 * 1 * 5 * 131 * 4
    bad = good_problem(seq_q=2, seq_k=1000)
    bpr, bkeep = bad.to_c()
    assert lib.polar_attn_decode_workspace_bytes(ctypes.byref(bpr), 0) == 0
    o = outputs()
    # seq_q != 1 and fp32 are not decode problems
    assert lib.polar_attn_decode(ctypes.byref(bpr), fake(1), fake(2), fake(3), 0, fake(4), 1 << 20, ctypes.byref(o),
                                 None) == 3
    f32 = good_problem(seq_q=1, seq_k=1000, dtype=pa.POLAR_F32)
    fpr, fkeep = f32.to_c()
    assert lib.polar_attn_decode(ctypes.byref(fpr), fake(1), fake(2), fake(3), 0, fake(4), 1 << 20, ctypes.byref(o),
                                 None) == 3
    # workspace missing / too small / misaligned; too many splits
    assert lib.polar_attn_decode(ctypes.byref(pr), fake(1), fake(2), fake(3), 4, None, 0, ctypes.byref(o), None) == 6
    need = lib.polar_attn_decode_workspace_bytes(ctypes.byref(pr), 4)
    assert lib.polar_attn_decode(ctypes.byref(pr), fake(1), fake(2), fake(3), 4, fake(4), need - 1, ctypes.byref(o),
                                 None) == 6
    assert lib.polar_attn_decode(ctypes.byref(pr), fake(1), fake(2), fake(3), 4, ctypes.c_void_p(FAKE + 4 * (1 << 34) + 4),
                                 need, ctypes.byref(o), None) == 5
    assert lib.polar_attn_decode(ctypes.byref(pr), fake(1), fake(2), fake(3), 1001, fake(4), 1 << 30, ctypes.byref(o),
                                 None) == 2
    # workspace overlapping an output
    assert lib.polar_attn_decode(ctypes.byref(pr), fake(1), fake(2), fake(3), 4, fake(10), need, ctypes.byref(o),
                                 None) == 7
    # an empty batch: split count and workspace queries and the call itself are fine
    empty = good_problem(batch=0, seq_q=1, seq_k=1000, head_dim=128)
    epr, ekeep = empty.to_c()
    assert lib.polar_attn_decode_num_splits(ctypes.byref(epr), 0) == 1
    assert lib.polar_attn_decode_workspace_bytes(ctypes.byref(epr), 0) == 0
    assert lib.polar_attn_decode(ctypes.byref(epr), None, None, None, 0, None, 0,
                                 ctypes.byref(pa.PolarOutputs(None, None, None, None, None)), None) == 0
    # merge
    assert lib.polar_attn_merge(ctypes.byref(pr), None, 4, ctypes.byref(o), None) == 1
    assert lib.polar_attn_merge(ctypes.byref(pr), fake(4), 0, ctypes.byref(o), None) == 2
    assert lib.polar_attn_merge(ctypes.byref(pr), fake(10), 4, ctypes.byref(o), None) == 7


def test_decode_noalloc_validation(lib):
    """The no-allocation decode checks like polar_attn_decode, and rejects partials beyond
    its fixed array with POLAR_ERR_WORKSPACE, before any HIP call."""
    assert pa.NOALLOC_SCRATCH_BYTES == int(
        eval(re.search(r"#define POLAR_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
             .expand(r"\1 << \2")))
    o = outputs()
    big = good_problem(batch=64, heads=8, kv_heads=8, seq_q=1, seq_k=64, head_dim=128)
    pr, keep = big.to_c()
    need = lib.polar_attn_decode_workspace_bytes(ctypes.byref(pr), 64)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    assert lib.polar_attn_decode_noalloc(ctypes.byref(pr), fake(1), fake(2), fake(3), 64, ctypes.byref(o), None) == 6
    # the other checks are those of polar_attn_decode
    bad = good_problem(seq_q=2, seq_k=1000)
    bpr, bkeep = bad.to_c()
    assert lib.polar_attn_decode_noalloc(ctypes.byref(bpr), fake(1), fake(2), fake(3), 0, ctypes.byref(o), None) == 3
    ok = good_problem(seq_q=1, seq_k=1000, head_dim=128)
    opr, okeep = ok.to_c()
    assert lib.polar_attn_decode_noalloc(ctypes.byref(opr), None, fake(2), fake(3), 4, ctypes.byref(o), None) == 1
    assert lib.polar_attn_decode_noalloc(ctypes.byref(opr), fake(1), fake(2), fake(3), 1001, ctypes.byref(o),
                                         None) == 2
    assert lib.polar_attn_decode_noalloc(ctypes.byref(opr), fake(10), fake(2), fake(3), 4, ctypes.byref(o),
                                         None) == 7
    empty = good_problem(batch=0, seq_q=1, seq_k=1000, head_dim=128)
    epr, ekeep = empty.to_c()
    assert lib.polar_attn_decode_noalloc(ctypes.byref(epr), None, None, None, 0,
                                         ctypes.byref(pa.PolarOutputs(None, None, None, None, None)), None) == 0


def paged(num_blocks=64, block_size=16, max_blocks=64, table=None, lens=None, kp=None, vp=None):
    return pa.PolarPagedKV(fake(2) if kp is None else kp, fake(3) if vp is None else vp,
                           fake(5) if table is None else table, fake(6) if lens is None else lens,
                           num_blocks, block_size, max_blocks)


def test_paged_decode_validation(lib):
    prob = good_problem(batch=2, heads=8, kv_heads=2, seq_q=1, seq_k=1000, causal=False, head_dim=128)
    pr, keep = prob.to_c()
    kv = paged()
    nsplit = lib.polar_attn_decode_paged_num_splits
    wbytes = lib.polar_attn_decode_paged_workspace_bytes
    call = lib.polar_attn_decode_paged
    assert nsplit(ctypes.byref(pr), ctypes.byref(kv), 0) >= 1
    assert nsplit(ctypes.byref(pr), ctypes.byref(kv), 9) == 9
    assert nsplit(ctypes.byref(pr), ctypes.byref(kv), 1001) == 0
    assert nsplit(ctypes.byref(pr), None, 0) == 0
    assert wbytes(ctypes.byref(pr), ctypes.byref(kv), 3) == 2 * 8 * 1 * 3 * 131 * 4
    o = outputs()

    def run(kvx=None, q=None, splits=4, ws=None, wsb=1 << 26, prx=None, out=None):
        return call(ctypes.byref(pr if prx is None else prx), fake(1) if q is None else q,
                    None if kvx is False else ctypes.byref(kv if kvx is None else kvx), splits,
                    fake(4) if ws is None else ws, wsb, ctypes.byref(o if out is None else out), None)

    assert run(kvx=False) == 1
    assert run(q=ctypes.c_void_p(0)) == 1
    assert call(None, fake(1), ctypes.byref(kv), 4, fake(4), 1 << 26, ctypes.byref(o), None) == 1
    assert run(kvx=paged(table=ctypes.c_void_p(0))) == 1
    assert run(kvx=paged(lens=ctypes.c_void_p(0))) == 1
    assert run(kvx=paged(kp=ctypes.c_void_p(0))) == 1
    # block size must be a power of two in 1..1024; the table must cover seq_k
    for bs in (0, 3, 24, 2048):
        assert run(kvx=paged(block_size=bs, max_blocks=4096)) == 2, bs
    assert run(kvx=paged(num_blocks=0)) == 2
    assert run(kvx=paged(max_blocks=62)) == 2          # 62 * 16 < 1000
    assert run(kvx=paged(max_blocks=63)) != 2          # 63 * 16 >= 1000: passes this check
    assert run(splits=1001) == 2
    # decode problems only: one query per sequence, bf16
    two = good_problem(batch=2, heads=8, kv_heads=2, seq_q=2, seq_k=1000, causal=False, head_dim=128)
    tpr, tkeep = two.to_c()
    assert run(prx=tpr) == 3
    f32 = good_problem(batch=2, heads=8, kv_heads=2, seq_q=1, seq_k=1000, causal=False, head_dim=128,
                       dtype=pa.POLAR_F32)
    fpr, fkeep = f32.to_c()
    assert run(prx=fpr) == 3
    # alignment
    assert run(kvx=paged(table=ctypes.c_void_p(FAKE + 5 * (1 << 34) + 2))) == 5
    assert run(kvx=paged(kp=ctypes.c_void_p(FAKE + 2 * (1 << 34) + 8))) == 5
    assert run(ws=ctypes.c_void_p(FAKE + 4 * (1 << 34) + 4)) == 5
    # workspace missing or short
    need = wbytes(ctypes.byref(pr), ctypes.byref(kv), 4)
    assert run(ws=ctypes.c_void_p(0)) == 6
    assert run(wsb=need - 1) == 6
    # aliasing: workspace over the block table; an output over the lengths
    assert run(ws=fake(5)) == 7
    assert run(out=outputs(n_eff=fake(6))) == 7
    # an empty batch is accepted without pointers
    empty = good_problem(batch=0, heads=8, kv_heads=2, seq_q=1, seq_k=1000, causal=False, head_dim=128)
    epr, ekeep = empty.to_c()
    assert call(ctypes.byref(epr), None, ctypes.byref(paged(table=ctypes.c_void_p(0), lens=ctypes.c_void_p(0),
                                                             kp=ctypes.c_void_p(0), vp=ctypes.c_void_p(0))),
                0, None, 0, ctypes.byref(pa.PolarOutputs(None, None, None, None, None)), None) == 0


def test_grouped_auto_splits_count_group_chunks(lib):
    """A grouped workgroup serves up to 8 query heads of a group, so the automatic split
    count is sized by (batch x kv_heads x chunks) workgroups; it aims for 4096 split
    workgroups with one head per workgroup, 2048 with the grouped kernel over a contiguous
    cache and 6144 over a paged pool, with splits of at least 256 keys (2048 paged) and at
    most 128 splits."""
    mha = good_problem(batch=16, heads=8, kv_heads=8, seq_q=1, seq_k=1 << 20, causal=False, head_dim=128)
    gqa = good_problem(batch=16, heads=8, kv_heads=2, seq_q=1, seq_k=1 << 20, causal=False, head_dim=128)
    g3 = good_problem(batch=16, heads=6, kv_heads=2, seq_q=1, seq_k=1 << 20, causal=False, head_dim=128)
    few = good_problem(batch=2, heads=8, kv_heads=8, seq_q=1, seq_k=1 << 20, causal=False, head_dim=128)
    n = {}
    for name, prob in (("mha", mha), ("gqa", gqa), ("g3", g3), ("few", few)):
        pr, keep = prob.to_c()
        n[name] = lib.polar_attn_decode_num_splits(ctypes.byref(pr), 0)
    assert n["mha"] == 4096 // 128           # 128 (b, h) rows
    assert n["gqa"] == 2048 // 16 // 2 // 1  # 16 x 2 kv heads x 1 chunk of 4
    assert n["g3"] == -(-2048 // (16 * 6))   # group of 3 runs one head per workgroup
    assert n["few"] == 128                   # 4096 // 16 = 256 wanted, at most 128
    pr, keep = gqa.to_c()
    kv = paged(num_blocks=1 << 21, max_blocks=1 << 16)
    # paged: 6144 // 32 = 192 splits wanted, at most 128
    assert lib.polar_attn_decode_paged_num_splits(ctypes.byref(pr), ctypes.byref(kv), 0) == 128
    mid = good_problem(batch=16, heads=8, kv_heads=8, seq_q=1, seq_k=1 << 16, causal=False, head_dim=128)
    pr, keep = mid.to_c()
    kv = paged(num_blocks=1 << 16, max_blocks=1 << 12)
    # 6144 // 128 = 48 splits wanted, and each keeps at least 2048 of the 2^16 keys: 32
    assert lib.polar_attn_decode_paged_num_splits(ctypes.byref(pr), ctypes.byref(kv), 0) == (1 << 16) // 2048
    # at least 256 keys per split over a contiguous cache, 2048 over a paged pool
    short = good_problem(batch=2, heads=8, kv_heads=2, seq_q=1, seq_k=1000, causal=False, head_dim=128)
    pr, keep = short.to_c()
    assert lib.polar_attn_decode_num_splits(ctypes.byref(pr), 0) == 4
    assert lib.polar_attn_decode_paged_num_splits(ctypes.byref(pr), ctypes.byref(paged()), 0) == 1


def test_fwd_partial_validation(lib):
    prob = good_problem(seq_q=64, seq_k=64, head_dim=128, len_temp=[0.1, -0.1])
    pr, keep = prob.to_c()
    call = lib.polar_attn_fwd_partial
    assert call(ctypes.byref(pr), fake(1), fake(2), fake(3), 1000, None, 2, 0, None) == 1
    assert call(ctypes.byref(pr), None, fake(2), fake(3), 1000, fake(4), 2, 0, None) == 1
    for ns, sp in ((0, 0), (2, 2), (2, -1)):
        assert call(ctypes.byref(pr), fake(1), fake(2), fake(3), 1000, fake(4), ns, sp, None) == 2
    assert call(ctypes.byref(pr), fake(1), fake(2), fake(3), 63, fake(4), 2, 0, None) == 2      # < seq_q
    # tau = -0.1 is fine at 64 keys but lambda(1e6) = 1 - 0.1 ln 1e6 < 0
    assert call(ctypes.byref(pr), fake(1), fake(2), fake(3), 1000000, fake(4), 2, 0, None) == 4
    assert call(ctypes.byref(pr), fake(1), fake(2), fake(3), 1000, ctypes.c_void_p(FAKE + 4 * (1 << 34) + 2), 2, 0,
                None) == 5
    assert call(ctypes.byref(pr), fake(1), fake(2), fake(3), 1000, fake(2), 2, 0, None) == 7  # over k


def test_bwd_validation(lib):
    prob = good_problem(batch=2, heads=4, kv_heads=2, seq_q=48, seq_k=64, head_dim=128)
    pr, keep = prob.to_c()
    rows = 2 * 4 * 48
    up = lambda x: (x + 255) // 256 * 256
    # bf16: forward statistics (d + 3 fp32), w (d bf16), row constants (4 fp32), 256-byte
    # parts; 4 key tiles (one per (b, kv head)) under a causal mask want 2048 / 4 runs each,
    # clamped to 4 per query head (8): 8 partial dk and dv of 2 * 2 * 64 keys
    nk = 2 * 2 * 64
    ws = up(rows * 131 * 4) + up(rows * 128 * 2) + up(rows * 16) + 2 * up(8 * nk * 128 * 4)
    assert lib.polar_attn_bwd_workspace_bytes(ctypes.byref(pr)) == ws
    # enough key tiles (16 * 8 * 16 = 2048): no split, no partial sums
    big_pr, keep_big = good_problem(batch=16, heads=8, kv_heads=8, seq_q=2048, seq_k=2048, head_dim=128).to_c()
    r_big = 16 * 8 * 2048
    assert lib.polar_attn_bwd_workspace_bytes(ctypes.byref(big_pr)) == (
        up(r_big * 131 * 4) + up(r_big * 128 * 2) + up(r_big * 16))
    # full mask: 512 / 4 = 128 runs wanted, clamped to 8
    full_pr, keep_full = good_problem(batch=2, heads=4, kv_heads=2, seq_q=48, seq_k=64, head_dim=128,
                                      causal=False).to_c()
    assert lib.polar_attn_bwd_workspace_bytes(ctypes.byref(full_pr)) == ws
    pr32, keep32 = good_problem(batch=2, heads=4, kv_heads=2, seq_q=48, seq_k=64, head_dim=128,
                                dtype=pa.POLAR_F32).to_c()
    assert lib.polar_attn_bwd_workspace_bytes(ctypes.byref(pr32)) == rows * (128 + 4) * 4
    bad, keep2 = good_problem(head_dim=96).to_c()
    assert lib.polar_attn_bwd_workspace_bytes(ctypes.byref(bad)) == 0
    g = pa.PolarGrads(fake(20), fake(21), None, fake(22))
    call = lib.polar_attn_bwd

    def run(q=1, k=2, v=3, grads=g, dq=4, dk=5, dv=6, work=7, nbytes=ws, problem=pr):
        arg = lambda x: fake(x) if isinstance(x, int) else x
        gp = None if grads is None else ctypes.byref(grads)
        return call(ctypes.byref(problem), arg(q), arg(k), arg(v), gp, arg(dq), arg(dk), arg(dv), arg(work), nbytes,
                    None)

    assert run(problem=bad) == 3
    assert run(grads=None) == 1
    for name in ("q", "k", "v", "dq", "dk", "dv"):
        assert run(**{name: None}) == 1, name
    assert run(work=None) == 6
    assert run(nbytes=ws - 1) == 6
    odd = ctypes.c_void_p(FAKE + 8 * (1 << 34) + 8)  # 8-byte aligned only
    for name in ("q", "dq", "dk", "work"):
        assert run(**{name: odd}) == 5, name
    assert run(grads=pa.PolarGrads(odd, None, None, None)) == 5
    assert run(grads=pa.PolarGrads(None, ctypes.c_void_p(FAKE + 2), None, None)) == 5
    assert run(dk=1) == 7                    # dk over q
    assert run(work=20) == 7                 # workspace over d_direction
    assert run(dv=5) == 7                    # dv over dk
    bad_tau, keep3 = good_problem(len_temp=[0.0, -1.0]).to_c()
    assert run(problem=bad_tau) == 4
    # no batch: nothing to do, nothing checked past the problem
    empty, keep4 = good_problem(batch=0).to_c()
    assert run(problem=empty, q=None, k=None, v=None, dq=None, dk=None, dv=None, work=None, nbytes=0) == 0
    # no query rows: q, dq and the workspace may be NULL, k, v, dk, dv may not
    rows0, keep5 = good_problem(seq_q=0).to_c()
    assert lib.polar_attn_bwd_workspace_bytes(ctypes.byref(rows0)) == 0
    assert run(problem=rows0, dk=None, q=None, dq=None, work=None, nbytes=0) == 1
    # the fp32 path's (batch, head) grid dimension is limited to 65535 pairs
    big, keep6 = good_problem(batch=40000, heads=2, kv_heads=2, dtype=pa.POLAR_F32).to_c()
    assert run(problem=big) == 3


@pytest.mark.parametrize("variant,status", [
    (dict(temperature="log"), 0), (dict(window=-1), 4), (dict(temperature="train_ratio", train_len=1), 4),
    (dict(key_floor="soft"), 4),                      # a per-key floor without the floor
    (dict(window=16), 0),
])
def test_fwd_variant_validation(lib, variant, status):
    """Variant checks run before any launch; the calls that pass them fail on the fake
    output pointer overlap check instead (status 7), so nothing is launched."""
    prob = good_problem(variant=variant)
    out = outputs(direction=fake(2))  # overlaps k: the call stops at the alias check
    got = call_fwd(lib, prob, out=out)
    assert got == (7 if status == 0 else status)


def test_variant_enum_and_entry_checks(lib):
    def problem(**v):
        pr, keep = good_problem(null_bias=[0.0, 0.0]).to_c()
        var = pa.PolarVariant(v.get("t", 0), v.get("L", 2048), v.get("fl", 0), v.get("kf", 0), v.get("sat", 0),
                              v.get("w", 0))
        pr.variant = ctypes.pointer(var)
        return pr, (keep, var)

    def fwd(pr):
        o = outputs(direction=fake(2))
        return lib.polar_attn_fwd(ctypes.byref(pr), fake(1), fake(2), fake(3), ctypes.byref(o), None)

    for bad in (dict(t=3), dict(t=-1), dict(fl=3), dict(kf=3), dict(sat=2)):
        pr, keep = problem(**bad)
        assert fwd(pr) == 3, bad
    # ssmax needs tau >= 0
    pr, keep = problem(t=1)
    neg = (ctypes.c_float * 2)(0.5, -0.1)
    pr.len_temp = ctypes.cast(neg, ctypes.POINTER(ctypes.c_float))
    assert fwd(pr) == 4
    # a window needs the causal alignment in prefill
    pr, keep = problem(w=8)
    pr.causal = 0
    assert fwd(pr) == 3
    # the partial forward takes neither a window nor the data-adaptive level
    for v in (dict(w=8), dict(fl=2)):
        pr, keep = problem(**v)
        assert lib.polar_attn_fwd_partial(ctypes.byref(pr), fake(1), fake(2), fake(3), 0, fake(4), 2, 0, None) == 3
    # the public merge has no queries for the data-adaptive level
    pr, keep = problem(fl=2)
    o = outputs()
    assert lib.polar_attn_merge(ctypes.byref(pr), fake(4), 2, ctypes.byref(o), None) == 3
    # the backward takes the variants that change only per-row constants: a per-key floor,
    # a window or the data-adaptive level is unsupported; the others pass the variant check
    # and stop at the alias check (dq given k's address), so nothing is launched
    g = pa.PolarGrads(None, None, None, None)
    for v in (dict(kf=1), dict(kf=2), dict(w=4), dict(fl=2)):
        pr, keep = problem(**v)
        assert lib.polar_attn_bwd(ctypes.byref(pr), fake(1), fake(2), fake(3), ctypes.byref(g), fake(4), fake(5),
                                  fake(6), fake(7), 1 << 30, None) == 3, v
    for v in (dict(), dict(sat=1), dict(t=1), dict(t=2), dict(fl=1), dict(t=1, fl=1, sat=1)):
        pr, keep = problem(**v)
        assert lib.polar_attn_bwd(ctypes.byref(pr), fake(1), fake(2), fake(3), ctypes.byref(g), fake(2), fake(5),
                                  fake(6), fake(7), 1 << 30, None) == 7, v


def test_python_binding_checks():
    with pytest.raises(ValueError):
        good_problem(len_temp=[0.0]).to_c()
    assert issubclass(pa.PolarArgumentError, ValueError)


def test_build_compiles_for_gfx950():
    """build() produces a shared library with gfx950 device code (cross-compiled here)."""
    with open(pbuild.__file__) as f:
        src = f.read()
    assert 'ARCH = "gfx950"' in src and "-packed-fp32-ops" in src
