"""The C ABI on the host: the library loads, exports what the header declares,
and rejects bad arguments before touching a GPU (no kernel is launched here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import token_tree_verification_02_amd as tv
from token_tree_verification_02_amd import _lib
from token_tree_verification_02_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SIZE_MAX = (1 << 64) - 1


@pytest.fixture(scope="module")
def lib():
    return tv.load()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "tree_verify.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"tree_build", "tree_attention", "tree_verify_greedy", "tree_validate_host",
            "tree_attention_workspace_size", "tv_status_string", "tv_last_error", "tv_version"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.SIGNATURES)


def test_status_strings(lib):
    for code in range(6):
        assert lib.tv_status_string(code).decode()
    assert lib.tv_version() == 2


def test_host_validation_matches_oracle_on_all_small_trees():
    import itertools
    for n in range(1, 6):
        for choice in itertools.product(*[range(u) for u in range(1, n)]):
            parent = np.array([-1] + list(choice), np.int32)
            depth = W.depths_of(parent)
            assert tv.validate_host(parent, depth) == tv.TV_OK
            for u in range(n):          # one wrong depth anywhere is caught
                bad = depth.copy()
                bad[u] += 1
                assert (tv.validate_host(parent, bad) == tv.TV_OK) == oracle.validate_tree(parent, bad)


def test_host_validation_rejects(lib):
    p, d = W.expansion_tree([2, 2])
    for par, dep in [(np.r_[0, p[1:]], d), (np.r_[p[:3], 5, p[4:]], d), (p, np.r_[1, d[1:]]),
                     (np.r_[p[:2], -1, p[3:]], d)]:
        assert tv.validate_host(par, dep) == tv.TV_ETOPOLOGY
        assert tv.last_error()
    assert lib.tree_validate_host(0, p.ctypes.data, d.ctypes.data) == tv.TV_EINVAL
    assert lib.tree_validate_host(300, p.ctypes.data, d.ctypes.data) == tv.TV_EINVAL
    assert lib.tree_validate_host(7, None, d.ctypes.data) == tv.TV_EINVAL


def test_tree_build_argument_errors(lib):
    assert lib.tree_build(-1, 7, *([None] * 6), None) == tv.TV_EINVAL
    assert lib.tree_build(2, 0, *([None] * 6), None) == tv.TV_EINVAL
    assert lib.tree_build(2, 257, *([None] * 6), None) == tv.TV_EINVAL
    assert lib.tree_build(2, 7, *([None] * 6), None) == tv.TV_EINVAL      # null pointers
    assert lib.tree_build(0, 7, *([None] * 6), None) == tv.TV_OK          # empty batch: nothing to do


def desc(**kw):
    base = dict(B=8, n=21, Hq=32, Hkv=32, D=128, dtype=tv.TV_BF16, Lmax=1024)
    base.update(kw)
    paged = base.pop("paged", False)
    bs = base.pop("block_size", None)
    if paged:
        base.pop("Lmax")
        d = tv.attn_desc(base.pop("B"), base.pop("n"), base.pop("Hq"), base.pop("Hkv"), base.pop("D"),
                         base.pop("dtype"), paged=True, **base)
        if bs is not None:
            d.block_size = bs
        return d
    return tv.attn_desc(base.pop("B"), base.pop("n"), base.pop("Hq"), base.pop("Hkv"), base.pop("D"),
                        base.pop("dtype"), **base)


def test_workspace_size():
    assert tv.workspace_size(desc()) == 0                       # 256 (seq, head) pairs: no split
    d4 = desc(B=32, n=32, Hq=64, Hkv=8, paged=True, max_blocks=2048, num_blocks=41000)
    ws = tv.workspace_size(d4)
    assert ws > 0 and ws % 256 == 0
    for bad in (desc(Hq=30, Hkv=8), desc(D=96), desc(n=0), desc(n=300), desc(dtype=5), desc(Lmax=1000),
                desc(B=-1), desc(paged=True, max_blocks=10, num_blocks=10, block_size=8)):
        assert tv.workspace_size(bad) == SIZE_MAX


def call_attn(lib, d, ptr=0x100000, ws=None, wsb=0):
    p = [ptr] * 11
    return lib.tree_attention(ctypes.byref(d), *p, ws, wsb, None)


def test_attention_argument_errors(lib):
    assert call_attn(lib, desc(Hq=30, Hkv=8)) == tv.TV_EUNSUPPORTED
    assert call_attn(lib, desc(D=80)) == tv.TV_EUNSUPPORTED
    assert call_attn(lib, desc(dtype=3)) == tv.TV_EUNSUPPORTED
    assert call_attn(lib, desc(Lmax=24)) == tv.TV_EINVAL
    assert call_attn(lib, desc(paged=True, max_blocks=4, num_blocks=4, block_size=32)) == tv.TV_EUNSUPPORTED
    d = desc()
    assert lib.tree_attention(ctypes.byref(d), *([None] * 12), 0, None) == tv.TV_EINVAL   # null pointers
    assert call_attn(lib, d, ptr=0x100002) == tv.TV_EINVAL                                # misaligned
    d4 = desc(B=32, n=32, Hq=64, Hkv=8, paged=True, max_blocks=2048, num_blocks=41000)
    need = tv.workspace_size(d4)
    assert call_attn(lib, d4, ws=None, wsb=0) == tv.TV_EWORKSPACE
    assert call_attn(lib, d4, ws=0x100000, wsb=need - 1) == tv.TV_EWORKSPACE
    assert "workspace" in tv.last_error()
    assert lib.tree_attention(ctypes.byref(desc(B=0)), *([None] * 12), 0, None) == tv.TV_OK


def test_verify_argument_errors(lib):
    args = [0x100000] * 8
    assert lib.tree_verify_greedy(2, 7, 0, tv.TV_BF16, *args, None) == tv.TV_EINVAL
    assert lib.tree_verify_greedy(2, 0, 10, tv.TV_BF16, *args, None) == tv.TV_EINVAL
    assert lib.tree_verify_greedy(2, 300, 10, tv.TV_BF16, *args, None) == tv.TV_EINVAL
    assert lib.tree_verify_greedy(2, 7, 10, 9, *args, None) == tv.TV_EUNSUPPORTED
    assert lib.tree_verify_greedy(2, 7, 10, tv.TV_F32, *([None] * 8), None) == tv.TV_EINVAL
    assert lib.tree_verify_greedy(0, 7, 10, tv.TV_F32, *([None] * 8), None) == tv.TV_OK


def call_commit(lib, d, ptrs=None, new_len=0x300000):
    p = [0x100000, 0x100000, 0x100000, 0x200000, 0x100000, 0x100000, 0x100000, 0x100000] if ptrs is None else ptrs
    return lib.tree_commit_kv(ctypes.byref(d), *p, new_len, None, None)


def test_commit_argument_errors(lib):
    assert call_commit(lib, desc(D=80)) == tv.TV_EUNSUPPORTED
    assert call_commit(lib, desc(dtype=3)) == tv.TV_EUNSUPPORTED
    assert call_commit(lib, desc(Lmax=24)) == tv.TV_EINVAL
    assert call_commit(lib, desc(n=0)) == tv.TV_EINVAL
    assert call_commit(lib, desc(), new_len=None) == tv.TV_EINVAL                 # null output
    assert call_commit(lib, desc(), ptrs=[None] * 8) == tv.TV_EINVAL              # null inputs
    assert call_commit(lib, desc(paged=True, max_blocks=4, num_blocks=4),
                       ptrs=[0x100000, 0x100000, None] + [0x100000] * 5) == tv.TV_EINVAL   # no block table
    misaligned = [0x100008, 0x100000, 0x100000, 0x200000, 0x100000, 0x100000, 0x100000, 0x100000]
    assert call_commit(lib, desc(), ptrs=misaligned) == tv.TV_EINVAL
    assert call_commit(lib, desc(), new_len=0x200000) == tv.TV_EINVAL             # aliases prefix_len
    assert call_commit(lib, desc(B=8), new_len=0x200000 + 28) == tv.TV_EINVAL     # overlaps it
    assert "overlap" in tv.last_error()
    assert lib.tree_commit_kv(ctypes.byref(desc(B=0)), *([None] * 10), None) == tv.TV_OK


def test_stochastic_argument_errors(lib):
    ws = lib.tree_verify_stochastic_workspace_size
    # two fp32 rows per sequence, row statistics, then the sliced walk's two slots of 16
    # exchange records (16 tagged 64-bit words) per sequence
    assert ws(8, 21, 32000) == 8 * 2 * 32768 * 4 + 8 * 21 * 2 * 16 + 8 * 2 * 16 * 16 * 8
    assert ws(0, 5, 5) == 0
    assert ws(-1, 5, 5) == SIZE_MAX and ws(2, 5, 0) == SIZE_MAX and ws(2, 5, tv.TV_MSS_VMAX + 1) == SIZE_MAX
    assert ws(2, 0, 5) == SIZE_MAX and ws(2, 257, 5) == SIZE_MAX
    p = [0x100000] * 10
    call = lambda B, n, V, dt, ptrs=p, w=0x100000, wb=1 << 30, mode=0: lib.tree_verify_stochastic(
        B, n, V, dt, mode, *ptrs, w, wb, None)
    assert call(2, 7, 0, tv.TV_BF16) == tv.TV_EINVAL
    assert call(2, 7, tv.TV_MSS_VMAX + 1, tv.TV_BF16) == tv.TV_EINVAL
    assert call(2, 0, 10, tv.TV_BF16) == tv.TV_EINVAL
    assert call(2, 300, 10, tv.TV_BF16) == tv.TV_EINVAL
    assert call(2, 7, 10, 4) == tv.TV_EUNSUPPORTED
    assert call(2, 7, 10, tv.TV_F32, ptrs=[None] * 10) == tv.TV_EINVAL
    assert call(2, 7, 10, tv.TV_F32, w=None) == tv.TV_EWORKSPACE
    assert call(2, 7, 10, tv.TV_F32, wb=ws(2, 7, 10) - 1) == tv.TV_EWORKSPACE
    assert call(2, 7, 10, tv.TV_F32, mode=4) == tv.TV_EINVAL
    assert call(2, 7, 10, tv.TV_F32, mode=-1) == tv.TV_EINVAL
    assert call(2, 7, 10, tv.TV_F32, ptrs=[0x100004] + [0x100000] * 9) == tv.TV_EINVAL   # misaligned logits
    assert call(0, 7, 10, tv.TV_F32, ptrs=[None] * 10, w=None, wb=0) == tv.TV_OK


def test_stochastic_poll_limit(lib):
    """The bound on the sliced walk's waits: set and read back; a negative value is
    refused and leaves the limit alone."""
    prev = tv.stochastic_set_poll_limit(7)
    try:
        assert prev == 1 << 18
        assert tv.stochastic_set_poll_limit(0) == 7
        old = ctypes.c_int32(-5)
        assert lib.tree_verify_stochastic_set_poll_limit(-1, ctypes.byref(old)) == tv.TV_EINVAL
        assert old.value == -5
        assert lib.tree_verify_stochastic_set_poll_limit(3, None) == tv.TV_OK
        assert tv.stochastic_set_poll_limit(0) == 3
    finally:
        tv.stochastic_set_poll_limit(prev)


def test_construction_argument_errors(lib):
    P = [0x100000] * 9
    ex = lambda B, F, V, k, n_max, dt=tv.TV_BF16, ptrs=P: lib.tree_expand_topk(B, F, V, k, n_max, dt, *ptrs, None)
    assert ex(2, 0, 100, 2, 64) == tv.TV_EINVAL
    assert ex(2, 257, 100, 2, 64) == tv.TV_EINVAL
    assert ex(2, 3, 100, 0, 64) == tv.TV_EINVAL
    assert ex(2, 3, 100, tv.TV_TOPK_MAX + 1, 64) == tv.TV_EINVAL
    assert ex(2, 3, 4, 5, 64) == tv.TV_EINVAL                           # k > V
    assert ex(2, 3, 100, 2, tv.TV_NMAX + 1) == tv.TV_EINVAL
    assert ex(2, 3, 100, 2, 64, dt=7) == tv.TV_EUNSUPPORTED
    assert ex(2, 3, 100, 2, 64, ptrs=[None] * 9) == tv.TV_EINVAL
    assert ex(0, 3, 100, 2, 64, ptrs=[None] * 9) == tv.TV_OK
    mg = lambda B, M, Ld, n_max, ptrs=[0x100000] * 9: lib.tree_merge_drafts(B, M, Ld, n_max, *ptrs, None)
    assert mg(2, 0, 8, 64) == tv.TV_EINVAL
    assert mg(2, tv.TV_MERGE_MMAX + 1, 8, 64) == tv.TV_EINVAL
    assert mg(2, 3, 0, 64) == tv.TV_EINVAL
    assert mg(2, 3, tv.TV_NMAX, 64) == tv.TV_EINVAL
    assert mg(2, 3, 8, 0) == tv.TV_EINVAL
    assert mg(2, 3, 8, 64, ptrs=[None] * 9) == tv.TV_EINVAL
    assert mg(0, 3, 8, 64, ptrs=[None] * 9) == tv.TV_OK


def test_f16_descriptor_plans_like_bf16():
    for kw in (dict(), dict(B=32, n=32, Hq=64, Hkv=8, paged=True, max_blocks=2048, num_blocks=41000)):
        assert tv.workspace_size(desc(dtype=tv.TV_F16, **kw)) == tv.workspace_size(desc(dtype=tv.TV_BF16, **kw))



def test_fp8_cache_contract(lib):
    fp8 = dict(kv_dtype=tv.TV_FP8_E4M3, k_scale=0.01, v_scale=0.02)
    ok = desc(**fp8)                                                     # 21 rows per KV head
    assert tv.workspace_size(ok) != SIZE_MAX
    many = dict(B=32, n=32, Hq=64, Hkv=8)                                # 256 rows: the balanced schedule
    assert tv.workspace_size(desc(**many)) != SIZE_MAX
    assert tv.workspace_size(desc(**many, **fp8)) == SIZE_MAX            # fp8 is limited to 128 rows per KV head
    assert call_attn(lib, desc(**many, **fp8)) == tv.TV_EUNSUPPORTED
    assert tv.workspace_size(desc(B=32, n=16, Hq=64, Hkv=8, **fp8)) != SIZE_MAX   # 128 rows
    assert call_attn(lib, desc(dtype=tv.TV_F16, **fp8)) == tv.TV_EUNSUPPORTED
    assert call_attn(lib, desc(kv_dtype=tv.TV_FP8_E4M3, k_scale=0.0, v_scale=1.0)) == tv.TV_EINVAL
    assert call_attn(lib, desc(kv_dtype=9)) == tv.TV_EUNSUPPORTED
    assert call_commit(lib, desc(**fp8)) == tv.TV_EUNSUPPORTED


def test_noalloc_host_checks(lib):
    """tree_attention_noalloc refuses, before any HIP call, descriptors that are invalid or
    need more scratch than it holds; the limit covers the numbered workloads."""
    p = [0x100000] * 11
    call = lambda d: lib.tree_attention_noalloc(ctypes.byref(d), *p, None)
    assert call(desc(Hq=30, Hkv=8)) == tv.TV_EUNSUPPORTED
    big = desc(B=1, n=256, Hq=1024, Hkv=1)                    # 262144 rows per KV head
    assert tv.workspace_size(big) > tv.TV_NOALLOC_SCRATCH_BYTES
    assert call(big) == tv.TV_EWORKSPACE
    assert "scratch" in tv.last_error()
    for d in (desc(B=32, n=32, Hq=64, Hkv=8, paged=True, max_blocks=2048, num_blocks=41000),
              desc(B=16, n=64, Hq=64, Hkv=8, Lmax=2048), desc(B=64, n=128, Hq=32, Hkv=8, Lmax=8192),
              desc(B=8, n=21, Hq=32, Hkv=32, Lmax=1024)):
        assert tv.workspace_size(d) <= tv.TV_NOALLOC_SCRATCH_BYTES
    assert lib.tree_attention_noalloc(ctypes.byref(desc(B=0)), *([None] * 11), None) == tv.TV_OK


def test_noalloc_limit_matches_header():
    src = open(os.path.join(ROOT, "include", "tree_verify.h")).read()
    m = re.search(r"#define TV_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m, "TV_NOALLOC_SCRATCH_BYTES not found"
    assert int(m.group(1)) << int(m.group(2)) == tv.TV_NOALLOC_SCRATCH_BYTES
