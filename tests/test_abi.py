"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments on the host (before any HIP
call) with the documented status codes."""
import ctypes
import os
import re
import subprocess

import pytest

from long_context_prefill_swa_amd import build as hipbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "orthros.h")

OK, EINVAL, EUNSUP, ECAP, EWS, EHIP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
FAKE = 0x100000   # 16-byte aligned, never dereferenced by host validation


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hipbuild.LIB):
        hipbuild.build()
    import long_context_prefill_swa_amd as m
    return m.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*\*?\s*"
                                 r"(orthros_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("orthros_kv_append", "orthros_swa_prefill",
              "orthros_global_xattn", "orthros_decode_pair",
              "orthros_kv_append_paged", "orthros_decode_pair_paged",
              "orthros_layer_forward", "orthros_layer_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", hipbuild.LIB],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (orthros_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(L, n)


def test_abi_version_and_strerror(L):
    assert L.orthros_abi_version() == 7
    for code in (OK, EINVAL, EUNSUP, ECAP, EWS, EHIP):
        assert L.orthros_strerror(code)
    assert b"unknown" in L.orthros_strerror(42)


def last(L):
    return L.orthros_last_error().decode()


def swa(L, **kw):
    a = dict(q=FAKE, al=FAKE, be=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, T=64,
             Hq=4, Hkv=2, D=128, cap=64, W=16, hmap=None, dtype=BF16)
    a.update(kw)
    return L.orthros_swa_prefill(a["q"], a["al"], a["be"], a["k"], a["v"],
                                 a["o"], a["B"], a["T"], a["Hq"], a["Hkv"],
                                 a["D"], a["cap"], a["W"], a["hmap"],
                                 a["dtype"], None)


def hmap(vals):
    arr = (ctypes.c_int32 * len(vals))(*vals)
    return ctypes.cast(arr, ctypes.c_void_p), arr


@pytest.mark.parametrize("kw,code,needle", [
    (dict(dtype=7), EUNSUP, "dtype"),
    (dict(D=0), EUNSUP, "head dimension"),
    (dict(D=257), EUNSUP, "head dimension"),
    (dict(D=15), EUNSUP, "even"),
    (dict(W=0), EINVAL, "window"),
    (dict(Hq=6, Hkv=4), EINVAL, "multiple"),
    (dict(Hq=0), EINVAL, "head counts"),
    (dict(Hq=129, Hkv=1), EINVAL, "head counts"),
    (dict(cap=63), EINVAL, "cap"),
    (dict(T=-1), EINVAL, "negative"),
    (dict(q=None), EINVAL, "null"),
    (dict(o=None), EINVAL, "null"),
])
def test_swa_prefill_rejects(L, kw, code, needle):
    assert swa(L, **kw) == code
    assert needle in last(L)


def test_swa_prefill_head_map_checked(L):
    p, keep = hmap([0, 1, 2, 1])       # KV head 2 does not exist (Hkv=2)
    assert swa(L, hmap=p) == EINVAL and "head_map[2]" in last(L)
    p, keep = hmap([0, 1, 1, 1])       # a valid uneven map passes validation
    assert swa(L, hmap=p, B=0) == OK


def test_zero_sized_calls_are_no_ops(L):
    # return before any HIP call: valid even without a GPU
    assert swa(L, B=0) == OK
    assert swa(L, T=0) == OK
    assert L.orthros_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, 2, 128,
                               64, BF16, None) == OK
    assert L.orthros_global_xattn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 10,
                                  0, 4, 2, 128, 64, None, BF16, None, 0,
                                  None) == OK


def test_kv_append_rejects(L):
    assert L.orthros_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 65, 2, 128,
                               64, BF16, None) == ECAP
    assert L.orthros_kv_append(FAKE, FAKE, None, FAKE, FAKE, 1, 4, 2, 128,
                               64, BF16, None) == EINVAL
    assert L.orthros_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 0, 128,
                               64, BF16, None) == EINVAL
    assert L.orthros_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 128,
                               64, 3, None) == EUNSUP


def test_global_xattn_rejects(L):
    args = [FAKE] * 6 + [1, 100, 1, 4, 2, 128, 101, None, BF16]
    # split-KV path needs a workspace
    assert L.orthros_global_xattn(*args, None, 0, None) == EWS
    assert "workspace" in last(L)
    need = L.orthros_workspace_bytes(1, 1, 4, 2, 128, 1, 101, None)
    assert need > 0
    assert L.orthros_global_xattn(*args, FAKE, need - 1, None) == EWS
    bad = [FAKE] * 6 + [1, 100, 1, 4, 2, 128, 100, None, BF16]   # cap < T
    assert L.orthros_global_xattn(*bad, FAKE, need, None) == EINVAL


def decode(L, **kw):
    a = dict(B=2, Hq=4, Hkv=2, D=128, cap=100, max_len=50, W=16, ws=None,
             ws_bytes=0, dtype=BF16, cl=FAKE)
    a.update(kw)
    ptrs = [FAKE] * 10
    return L.orthros_decode_pair(*ptrs[:10], a["cl"], FAKE, FAKE, a["B"],
                                 a["Hq"], a["Hkv"], a["D"], a["cap"],
                                 a["max_len"], a["W"], None, a["dtype"],
                                 a["ws"], a["ws_bytes"], None)


def test_decode_pair_rejects(L):
    assert decode(L, max_len=101) == ECAP
    assert decode(L, max_len=0) == EINVAL
    assert decode(L, W=0) == EINVAL
    assert decode(L, cl=None) == EINVAL
    assert decode(L) == EWS
    assert decode(L, B=0) == OK


def test_workspace_bytes(L):
    def ws(*a):
        return L.orthros_workspace_bytes(*a, None)
    assert ws(9, 1, 4, 2, 128, 1, 100) == 0            # unknown op
    assert ws(2, 0, 4, 2, 128, 1, 100) == 0            # empty batch
    d1 = ws(2, 64, 32, 8, 128, 1, 33024)
    d2 = ws(2, 64, 32, 8, 128, 1, 66048)
    assert 0 < d1 < d2
    # global pass with many output rows uses no workspace (banded kernel)
    assert ws(1, 4, 32, 8, 128, 2048, 8192) == 0
    # non-128 head dimensions run the generic kernel without workspace
    assert ws(1, 1, 2, 2, 16, 1, 64) == 0
    # no map and Hq not a multiple of Hkv: invalid
    assert ws(1, 1, 5, 2, 128, 1, 100) == 0


def test_workspace_counter_bytes(L):
    """The arrival counters: one int32 per (batch entry, head group) and one
    per batch entry, padded to 256 bytes, at the front of the workspace;
    they depend on B and the head grouping, not on the lengths."""
    def cb(*a, m=None):
        return L.orthros_workspace_counter_bytes(*a, m)
    # 32 query heads on 8 KV heads: a decode pair has 2 rows per query head,
    # so each KV head's 4 heads form one group (8 rows): 8 groups
    assert cb(2, 64, 32, 8, 128, 1, 33024) == 64 * 9 * 4
    assert cb(2, 64, 32, 8, 128, 1, 66048) == 64 * 9 * 4
    assert cb(2, 1, 32, 8, 128, 1, 131072) == 256
    # one output row of 32 heads: 8 groups of 4 rows
    assert cb(1, 1, 32, 8, 128, 1, 131072) == 256
    assert cb(1, 100, 32, 8, 128, 1, 4096) == (100 * 9 * 4 + 255) // 256 * 256
    for a in ((9, 1, 4, 2, 128, 1, 100), (2, 0, 4, 2, 128, 1, 100),
              (1, 4, 32, 8, 128, 2048, 8192), (1, 1, 5, 2, 128, 1, 100)):
        assert cb(*a) == 0 and L.orthros_workspace_bytes(*a, None) == 0
    for a in ((2, 64, 32, 8, 128, 1, 33024), (1, 1, 32, 8, 128, 1, 131072)):
        assert 0 < cb(*a) < L.orthros_workspace_bytes(*a, None)


def imap(m):
    return (ctypes.c_int32 * len(m))(*m)


@pytest.mark.parametrize("Hq,Hkv,hm", [
    (6, 3, [0, 0, 0, 1, 2, 2]),       # uneven: 3, 1, 2 heads per KV head
    (5, 2, [0, 1, 1, 0, 1]),          # Hq not a multiple of Hkv
    (8, 2, [1, 1, 1, 1, 1, 1, 1, 0]),  # 7 heads on one KV head
])
def test_workspace_bytes_follows_the_head_map(L, Hq, Hkv, hm):
    """The size the query returns for a map is the size the calls with that
    map check against: one byte less is rejected with EWORKSPACE, the size
    itself passes the workspace check (the call then fails only at the
    launch, with no GPU here)."""
    m = imap(hm)
    for op in (1, 2):
        need = L.orthros_workspace_bytes(op, 2, Hq, Hkv, 128, 1, 300, m)
        assert need > 0
        if op == 1:
            def call(nb):
                return L.orthros_global_xattn(
                    *[FAKE] * 6, 2, 299, 1, Hq, Hkv, 128, 300, m, BF16,
                    FAKE, nb, None)
        else:
            def call(nb):
                return L.orthros_decode_pair(
                    *[FAKE] * 10, FAKE, FAKE, FAKE, 2, Hq, Hkv, 128, 400, 300,
                    16, m, BF16, FAKE, nb, None)
        assert call(need - 1) == EWS, last(L)
        assert call(need) in (OK, EHIP), last(L)
    # the default grouping's size can be smaller than the map's
    if Hq % Hkv == 0:
        assert L.orthros_workspace_bytes(2, 2, Hq, Hkv, 128, 1, 300, None) <= \
            L.orthros_workspace_bytes(2, 2, Hq, Hkv, 128, 1, 300, m)
    bad = imap([0] * (Hq - 1) + [Hkv])    # entry out of range
    assert L.orthros_workspace_bytes(2, 2, Hq, Hkv, 128, 1, 300, bad) == 0


def test_workspace_query_keeps_the_last_error(L):
    assert decode(L, W=0) == EINVAL
    msg = last(L)
    assert msg
    L.orthros_workspace_bytes(2, 2, 4, 2, 128, 1, 100, imap([0, 0, 0, 5]))
    assert last(L) == msg


def paged_append(L, **kw):
    a = dict(n_pages=16, page_size=64, max_pages=4, B=2, n=10, Hkv=2, D=128,
             dtype=BF16, bt=FAKE, cl=FAKE)
    a.update(kw)
    return L.orthros_kv_append_paged(FAKE, FAKE, a["n_pages"], a["page_size"],
                                     a["bt"], a["max_pages"], a["cl"], FAKE,
                                     FAKE, a["B"], a["n"], a["Hkv"], a["D"],
                                     a["dtype"], None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(page_size=48), EINVAL, "power of two"),
    (dict(page_size=16), EINVAL, "power of two"),
    (dict(page_size=1 << 17), EINVAL, "power of two"),
    (dict(n_pages=0), EINVAL, "n_pages"),
    (dict(max_pages=0), EINVAL, "max_pages"),
    (dict(bt=None), EINVAL, "null"),
    (dict(cl=None), EINVAL, "null"),
    (dict(n=257), ECAP, "max_pages"),
    (dict(dtype=5), EUNSUP, "dtype"),
    (dict(B=-1), EINVAL, "negative"),
])
def test_kv_append_paged_rejects(L, kw, code, needle):
    assert paged_append(L, **kw) == code
    assert needle in last(L)


def test_kv_append_paged_zero_sized(L):
    assert paged_append(L, B=0) == OK
    assert paged_append(L, n=0) == OK


def paged_decode(L, **kw):
    a = dict(n_pages=16, page_size=64, max_pages=4, B=2, Hq=4, Hkv=2, D=128,
             max_len=200, W=16, dtype=BF16, ws=None, ws_bytes=0, bt=FAKE,
             cl=FAKE)
    a.update(kw)
    return L.orthros_decode_pair_paged(
        *([FAKE] * 10), a["n_pages"], a["page_size"], a["bt"],
        a["max_pages"], a["cl"], FAKE, FAKE, a["B"], a["Hq"], a["Hkv"],
        a["D"], a["max_len"], a["W"], None, a["dtype"], a["ws"],
        a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(dtype=F32), EUNSUP, "bf16"),
    (dict(D=64), EUNSUP, "bf16"),
    (dict(page_size=100), EINVAL, "power of two"),
    (dict(max_len=257), ECAP, "max_pages"),
    (dict(max_len=0), EINVAL, "max_len_after"),
    (dict(W=0), EINVAL, "window"),
    (dict(bt=None), EINVAL, "null"),
    (dict(cl=None), EINVAL, "null"),
    (dict(Hq=6, Hkv=4), EINVAL, "multiple"),
    (dict(), EWS, "workspace"),
])
def test_decode_pair_paged_rejects(L, kw, code, needle):
    assert paged_decode(L, **kw) == code
    assert needle in last(L)


def test_decode_pair_paged_workspace_matches_contiguous(L):
    need = L.orthros_workspace_bytes(2, 2, 4, 2, 128, 1, 200, None)
    assert need > 0
    assert paged_decode(L, ws=FAKE, ws_bytes=need - 16) == EWS
    assert paged_decode(L, B=0) == OK


def layer(L, ws_bytes=None, **kw):
    a = dict(B=1, T=64, T_out=1, d_model=256, Hq=4, Hkv=2, D=128, cap=64,
             W=16, x=FAKE, y=FAKE)
    a.update(kw)
    need = L.orthros_layer_workspace_bytes(a["B"], a["T"], a["T_out"],
                                           a["d_model"], a["Hq"], a["Hkv"],
                                           a["D"])
    return L.orthros_layer_forward(
        a["x"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        FAKE, a["y"], a["B"], a["T"], a["T_out"], a["d_model"], a["Hq"],
        a["Hkv"], a["D"], a["cap"], a["W"], FAKE,
        need if ws_bytes is None else ws_bytes, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(T_out=65), EINVAL, "T_out"),
    (dict(T=0), EINVAL, "T_out"),
    (dict(d_model=0), EINVAL, "d_model"),
    (dict(Hq=6, Hkv=4), EINVAL, "heads"),
    (dict(D=15), EUNSUP, "head dimension"),
    (dict(W=0), EINVAL, "window"),
    (dict(cap=63), EINVAL, "cap"),
    (dict(x=None), EINVAL, "null"),
    (dict(y=None), EINVAL, "null"),
    (dict(ws_bytes=1000), EWS, "workspace"),
])
def test_layer_forward_rejects(L, kw, code, needle):
    assert layer(L, **kw) == code
    assert needle in last(L)


def test_layer_workspace_covers_the_intermediates(L):
    T, T_out, Hq, Hkv, D = 1000, 3, 8, 2, 128
    need = L.orthros_layer_workspace_bytes(1, T, T_out, 512, Hq, Hkv, D)
    inter = 2 * ((T + T_out) * Hq * D * 2) + 2 * (T * Hkv * D * 2)
    assert need >= inter + (64 << 20)
    assert L.orthros_layer_workspace_bytes(1, 10, 11, 512, Hq, Hkv, D) == 0
    assert layer(L, B=0) == OK


def bwd(L, ws_bytes=None, **kw):
    a = dict(B=1, T=64, T_out=2, Hq=4, Hkv=2, D=128, cap=64, W=16, hmap=None,
             dtype=BF16, q=FAKE)
    a.update(kw)
    need = L.orthros_backward_workspace_bytes(a["B"], a["T"], a["T_out"],
                                              a["Hq"], a["Hkv"], a["D"])
    return L.orthros_attn_backward(
        a["q"], *([FAKE] * 19), a["B"], a["T"], a["T_out"], a["Hq"],
        a["Hkv"], a["D"], a["cap"], a["W"], a["hmap"], a["dtype"], FAKE,
        need if ws_bytes is None else ws_bytes, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(dtype=F32), EUNSUP, "bf16"),
    (dict(D=64), EUNSUP, "D = 128"),
    (dict(T_out=65), EINVAL, "T_out"),
    (dict(W=0), EINVAL, "window"),
    (dict(cap=63), EINVAL, "cap"),
    (dict(Hq=32, Hkv=2), EUNSUP, "query heads"),
    (dict(q=None), EINVAL, "null"),
    (dict(ws_bytes=100), EWS, "workspace"),
])
def test_attn_backward_rejects(L, kw, code, needle):
    assert bwd(L, **kw) == code
    assert needle in last(L)


def test_attn_backward_kv_head_without_queries_rejected(L):
    p, keep = hmap([0, 0, 0, 0])       # KV head 1 has no query head
    assert bwd(L, hmap=p) == EUNSUP and "none" in last(L)
    assert bwd(L, B=0) == OK


# ---- binding-level size checks (CPU tensors: the size checks come before
# ---- the device checks, so they run without a GPU) -------------------------

def test_binding_checks_affine_and_length_sizes():
    import torch

    import long_context_prefill_swa_amd as lo
    B, T, Hq, Hkv, D = 1, 8, 4, 2, 128
    q = torch.zeros((B, T, Hq, D), dtype=torch.bfloat16)
    kc = torch.zeros((B, Hkv, T, D), dtype=torch.bfloat16)
    good = torch.zeros(Hq * D)
    short = torch.zeros(Hq * D - 1)
    with pytest.raises(ValueError, match="alpha must hold 512"):
        lo.orthros_swa_prefill(q, short, good, kc, kc, q, 4)
    with pytest.raises(ValueError, match="beta must hold 512"):
        lo.orthros_swa_prefill(q, good, short, kc, kc, q, 4)
    qx = torch.zeros((B, 1, Hq, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="alpha_x must hold 512"):
        lo.orthros_global_xattn(qx, short, good, kc, kc, qx, T - 1)
    qd = torch.zeros((B, Hq, D), dtype=torch.bfloat16)
    kn = torch.zeros((B, Hkv, D), dtype=torch.bfloat16)
    cl_bad = torch.zeros(B + 1, dtype=torch.int32)
    with pytest.raises(ValueError, match="cache_len must be int32 with B=1"):
        lo.orthros_decode_pair(qd, qd, good, good, good, good, kn, kn, kc, kc,
                               cl_bad, qd, qd, T, 4)
    with pytest.raises(ValueError, match="beta_x must hold 512"):
        lo.orthros_decode_pair(qd, qd, good, good, good, short, kn, kn, kc,
                               kc, torch.zeros(B, dtype=torch.int32), qd, qd,
                               T, 4)
    with pytest.raises(ValueError, match="cache_len must be int32"):
        lo.orthros_kv_append(kc, kc, torch.zeros(B, dtype=torch.int64),
                             torch.zeros((B, 2, Hkv, D), dtype=torch.bfloat16),
                             torch.zeros((B, 2, Hkv, D), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="head_map must have Hq=4"):
        lo.orthros_workspace_bytes(lo.ORTHROS_OP_DECODE_PAIR, B, Hq, Hkv, D, 1,
                                   T, head_map=[0, 1])


def test_binding_checks_block_table():
    import torch

    import long_context_prefill_swa_amd as lo
    pool = torch.zeros((4, 2, 32, 128), dtype=torch.bfloat16)
    kn = torch.zeros((1, 1, 2, 128), dtype=torch.bfloat16)
    cl = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="block_table must be int32"):
        lo.orthros_kv_append_paged(pool, pool,
                                   torch.zeros((1, 2), dtype=torch.int64), cl,
                                   kn, kn)
    with pytest.raises(ValueError, match="block_table must be a"):
        lo.orthros_kv_append_paged(pool, pool,
                                   torch.zeros(2, dtype=torch.int32), cl,
                                   kn, kn)


def test_noalloc_decode_pair_rejects_sizes_beyond_its_scratch(L):
    """Sizes whose split-KV scratch exceeds the static array are rejected on
    the host (EWORKSPACE), before anything is launched."""
    limit = 64 << 20
    assert L.orthros_workspace_bytes(2, 64, 32, 8, 128, 1, 200000, None) > limit
    rc = L.orthros_decode_pair_noalloc(*[FAKE] * 10, FAKE, FAKE, FAKE, 64, 32,
                                       8, 128, 200001, 200000, 2048, None,
                                       BF16, None)
    assert rc == EWS
    assert "no-allocation" in last(L)
    # counters beyond their fixed region: 2048 entries x (8 groups + 1)
    # int32 = 72 KiB, while the partials alone would fit
    assert L.orthros_workspace_counter_bytes(2, 2048, 8, 8, 128, 1, 100,
                                             None) > 64 << 10
    assert L.orthros_workspace_bytes(2, 2048, 8, 8, 128, 1, 100, None) < limit
    rc = L.orthros_decode_pair_noalloc(*[FAKE] * 10, FAKE, FAKE, FAKE, 2048, 8,
                                       8, 128, 101, 100, 16, None, BF16, None)
    assert rc == EWS
    assert "counters" in last(L)
    # ordinary argument errors come first, as in orthros_decode_pair
    assert L.orthros_decode_pair_noalloc(*[FAKE] * 10, FAKE, FAKE, FAKE, 2, 4,
                                         2, 128, 100, 101, 16, None, BF16,
                                         None) == ECAP
