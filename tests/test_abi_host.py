"""Host-side checks of the C ABI (no GPU needed): exports, argument validation, host helpers.

Every call here fails validation before the library makes any HIP call, so the fake device addresses used are
never dereferenced or launched on.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

import differential_attention_fwd_amd as da
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "diffattn.h")

OK, E_NULL, E_SHAPE, E_UNSUP, E_ALIGN, E_LAYER, E_LAMBDA, E_WS, E_ALIAS, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
BF16, F32 = 0, 1

# Fake, 16-byte aligned, widely separated addresses (never touched: every case below fails validation).
A = [0x10000000 * (i + 1) for i in range(8)]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(da.LIB_PATH):
        from differential_attention_fwd_amd import build
        build.build()
    return da.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(diffattn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(da.EXPORTS), names
    nm = subprocess.run(["nm", "-D", "--defined-only", da.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)", nm))
    for n in names:
        assert n in exported, f"{n} not exported"
        assert hasattr(lib, n)


def test_abi_version(lib):
    assert da.diffattn_abi_version() == 1


def test_lambda_init_matches_oracle(lib):
    for layer in range(1, 40):
        assert da.diffattn_lambda_init(layer) == pytest.approx(oracle.lambda_init(layer), abs=1e-15)
    assert da.diffattn_lambda_init(1) == pytest.approx(0.2, abs=1e-15)
    assert math.isnan(da.diffattn_lambda_init(0)) and math.isnan(da.diffattn_lambda_init(-3))


def test_status_strings(lib):
    seen = set()
    for s in range(0, -10, -1):
        msg = da.status_str(s)
        assert msg and msg != "unknown status"
        seen.add(msg)
    assert len(seen) == 10
    assert da.status_str(7) == "unknown status"


def fwd(lib, q1=A[0], k1=A[1], q2=A[2], k2=A[3], v=A[4], out=A[5], B=1, H=2, N=64, d=64, dtype=BF16, lam=0.5,
        layer=1, causal=1):
    return lib.diffattn_fwd(q1, k1, q2, k2, v, out, B, H, N, d, dtype, lam, layer, causal, None)


def dec(lib, q1=A[0], k1=A[1], q2=A[2], k2=A[3], v=A[4], out=A[5], B=2, H=2, L=100, d=64, dtype=BF16, lam=0.8,
        layer=1, causal=1, ws=A[6], ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.diffattn_decode_workspace_bytes(B, H, L, d)
    return lib.diffattn_decode(q1, k1, q2, k2, v, out, B, H, L, d, dtype, lam, layer, causal, ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    (dict(q1=None), E_NULL), (dict(k2=None), E_NULL), (dict(out=None), E_NULL),
    (dict(B=-1), E_SHAPE), (dict(N=-5), E_SHAPE), (dict(N=(1 << 23) + 1), E_SHAPE), (dict(H=1 << 40), E_SHAPE),
    (dict(d=32), E_UNSUP), (dict(d=128), E_UNSUP), (dict(dtype=7), E_UNSUP), (dict(dtype=F32, d=16), E_UNSUP),
    (dict(q2=A[2] + 8), E_ALIGN), (dict(out=A[5] + 2), E_ALIGN),
    (dict(layer=-1), E_LAYER), (dict(lam=float("nan")), E_LAMBDA), (dict(lam=float("inf")), E_LAMBDA),
    (dict(out=A[4] + 64), E_ALIAS), (dict(out=A[0]), E_ALIAS), (dict(out=A[3] - 64), E_ALIAS),
    (dict(N=0), OK), (dict(B=0), OK), (dict(H=0, q1=None), OK),
])
def test_fwd_validation(lib, case, expect):
    assert fwd(lib, **case) == expect


@pytest.mark.parametrize("case,expect", [
    (dict(L=0), E_SHAPE), (dict(L=-1), E_SHAPE), (dict(v=None), E_NULL), (dict(d=8), E_UNSUP),
    (dict(ws=None), E_WS), (dict(ws_bytes=16), E_WS), (dict(ws=A[6] + 4), E_ALIGN),
    (dict(ws=A[4]), E_ALIAS), (dict(out=A[1]), E_ALIAS), (dict(layer=-2), E_LAYER),
    (dict(lam=float("-inf")), E_LAMBDA), (dict(B=0), OK),
])
def test_decode_validation(lib, case, expect):
    assert dec(lib, **case) == expect


def test_workspace_bytes(lib):
    n = lib.diffattn_decode_workspace_bytes(64, 16, 8192, 64)
    assert n > 0 and n % 16 == 0
    # One (m, l, O[128]) state per map per split, per head: 1040 bytes per (head, split).
    assert n % (64 * 16 * 1040) == 0
    assert lib.diffattn_decode_workspace_bytes(1, 1, 1, 64) == 1040
    assert lib.diffattn_decode_workspace_bytes(2, 2, 0, 64) == 0
    assert lib.diffattn_decode_workspace_bytes(2, 2, 100, 8) == 0
    assert lib.diffattn_decode_workspace_bytes(0, 2, 100, 64) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(da, "_lib", None)
    monkeypatch.setattr(da, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        da.lib()


def test_oracle_is_not_imported_by_product():
    pkg = os.path.join(ROOT, "differential_attention_fwd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "oracle_diffattn" not in text, f


def fwd_heads(lib, lh=A[7], out=A[5], B=1, H=2, N=64, d=64, dtype=BF16, layer=1, causal=1):
    return lib.diffattn_fwd_heads(A[0], A[1], A[2], A[3], A[4], out, B, H, N, d, dtype, lh, layer, causal, None)


def dec_heads(lib, lh=A[7], out=A[5], ws=A[6], B=2, H=2, L=100, d=64, dtype=BF16, layer=1):
    n = lib.diffattn_decode_workspace_bytes(B, H, L, d)
    return lib.diffattn_decode_heads(A[0], A[1], A[2], A[3], A[4], out, B, H, L, d, dtype, lh, layer, 1, ws, n,
                                     None)


@pytest.mark.parametrize("case,expect", [
    (dict(lh=None), E_NULL), (dict(lh=A[7] + 2), E_ALIGN), (dict(lh=A[5] + 64), E_ALIAS), (dict(lh=A[5] - 4), E_ALIAS),
    (dict(N=0, lh=None), OK), (dict(H=0, lh=None), OK), (dict(layer=-1), E_LAYER), (dict(d=32), E_UNSUP),
])
def test_fwd_heads_validation(lib, case, expect):
    assert fwd_heads(lib, **case) == expect


@pytest.mark.parametrize("case,expect", [
    (dict(lh=None), E_NULL), (dict(lh=A[7] + 1), E_ALIGN), (dict(lh=A[6] + 16), E_ALIAS), (dict(lh=A[5]), E_ALIAS),
    (dict(B=0, lh=None), OK), (dict(L=0), E_SHAPE),
])
def test_decode_heads_validation(lib, case, expect):
    assert dec_heads(lib, **case) == expect


def test_lambda_heads_4_byte_alignment_is_enough(lib):
    # A per-head lambda array only needs 4-byte alignment; this call still fails, but later (on the output alias).
    assert fwd_heads(lib, lh=A[7] + 4, out=A[7]) == E_ALIAS


# B1 H2 N1000 takes 8 key splits (causal), so its calls need a workspace.
def fwd_split(lib, ws=A[6], ws_bytes=None, out=A[5], B=1, H=2, N=1000, d=64, dtype=BF16, lam=0.5, lh=None,
              layer=1):
    if ws_bytes is None:
        ws_bytes = lib.diffattn_fwd_split_workspace_bytes(B, H, N, d)
    return lib.diffattn_fwd_split(A[0], A[1], A[2], A[3], A[4], out, B, H, N, d, dtype, lam, lh, layer, 1, ws,
                                  ws_bytes, None)


def test_fwd_split_workspace_sizes(lib):
    # The plan (least modelled time among 1..16 splits) for the larger of the two masks sizes the workspace: 1040
    # bytes of partial state per row and split.  B1 H8 N1024: 4 splits causal, 1 not.
    assert lib.diffattn_fwd_split_workspace_bytes(1, 8, 1024, 64) == 8 * 1024 * 4 * 1040
    # B1 H1 N8192: 9 splits causal (29 key tiles each), 5 not
    assert lib.diffattn_fwd_split_workspace_bytes(1, 1, 8192, 64) == 8192 * 9 * 1040
    # B1 H1 N2049: 11 splits either way
    assert lib.diffattn_fwd_split_workspace_bytes(1, 1, 2049, 64) == 2049 * 11 * 1040
    # B1 H2 N64: too little work to gain from a merge -> no split, no workspace
    assert lib.diffattn_fwd_split_workspace_bytes(1, 2, 64, 64) == 0
    # B2 H8 N2048 (256 row tiles): splitting is modelled slower
    assert lib.diffattn_fwd_split_workspace_bytes(2, 8, 2048, 64) == 0
    # row tiles fill the 512 workgroup slots (B8 H8 N1024, B4 H12 N4096) -> no split; N <= 32: one key tile
    assert lib.diffattn_fwd_split_workspace_bytes(8, 8, 1024, 64) == 0
    assert lib.diffattn_fwd_split_workspace_bytes(4, 12, 4096, 64) == 0
    assert lib.diffattn_fwd_split_workspace_bytes(1, 1, 32, 64) == 0
    for bad in ((1, 1, 64, 8), (-1, 1, 64, 64), (1, 1, (1 << 23) + 1, 64)):
        assert lib.diffattn_fwd_split_workspace_bytes(*bad) == 0


@pytest.mark.parametrize("case,expect", [
    (dict(), OK), (dict(ws=None), E_WS), (dict(ws_bytes=1024), E_WS), (dict(ws=A[6] + 8), E_ALIGN),
    (dict(ws=A[4]), E_ALIAS), (dict(ws=A[5] - 64), E_ALIAS), (dict(out=A[0] + 128), E_ALIAS),
    (dict(dtype=F32), E_UNSUP), (dict(d=8), E_UNSUP), (dict(N=0), OK), (dict(B=-1), E_SHAPE),
    (dict(layer=-1), E_LAYER), (dict(lam=float("nan")), E_LAMBDA),
    (dict(B=4, H=12, N=4096, ws=None, ws_bytes=0), OK),   # fills the GPU without splits: no workspace needed
    (dict(lh=A[7] + 2), E_ALIGN), (dict(lh=A[5] + 4), E_ALIAS), (dict(lh=A[6] + 64), E_ALIAS),   # lambda per head
    (dict(lh=A[7], lam=float("nan"), out=A[0] + 128), E_ALIAS),   # lambda_heads: the scalar lambda is not checked
])
def test_fwd_split_validation(lib, case, expect):
    if expect == OK and case.get("N", 1) != 0:
        pytest.skip("valid calls would launch kernels (no GPU here)")
    assert fwd_split(lib, **case) == expect


def fwd_train(lib, saved=A[6], saved_bytes=None, out=A[5], B=1, H=2, N=64, d=64, dtype=BF16, lam=0.5, lh=None,
              layer=1):
    if saved_bytes is None:
        saved_bytes = lib.diffattn_train_saved_bytes(B, H, N, d)
    return lib.diffattn_fwd_train(A[0], A[1], A[2], A[3], A[4], out, B, H, N, d, dtype, lam, lh, layer, 1, saved,
                                  saved_bytes, None)


G = [0x80000000 + 0x10000000 * i for i in range(8)]   # more fake, widely separated device addresses


def bwd(lib, dq1=G[0], dlam=G[5], ws=G[6], ws_bytes=None, saved=A[6], B=1, H=2, N=64, d=64, dtype=BF16, lam=0.5,
        lh=None, layer=1):
    if ws_bytes is None:
        ws_bytes = lib.diffattn_bwd_workspace_bytes(B, H, N, d)
    return lib.diffattn_bwd(A[0], A[1], A[2], A[3], A[4], A[7], saved, dq1, G[1], G[2], G[3], G[4], dlam, B, H, N,
                            d, dtype, lam, lh, layer, 1, ws, ws_bytes, None)


def test_train_sizes(lib):
    assert lib.diffattn_train_saved_bytes(2, 3, 100, 64) == 2 * 3 * 100 * 1040
    assert lib.diffattn_train_saved_bytes(2, 3, 100, 8) == 0
    n = lib.diffattn_bwd_workspace_bytes(2, 3, 100, 64)
    assert n >= 2 * 3 * 100 * (256 + 16 + 4) and n % 256 == 0
    assert lib.diffattn_bwd_workspace_bytes(2, 3, 0, 64) == 0


@pytest.mark.parametrize("case,expect", [
    (dict(saved=None), E_NULL), (dict(saved_bytes=64), E_WS), (dict(saved=A[6] + 8), E_ALIGN),
    (dict(saved=A[4]), E_ALIAS), (dict(saved=A[5] + 64), E_ALIAS), (dict(dtype=F32), E_UNSUP), (dict(d=8), E_UNSUP),
    (dict(N=0), OK), (dict(lam=float("nan")), E_LAMBDA), (dict(layer=-1), E_LAYER), (dict(lh=A[7] + 2), E_ALIGN),
])
def test_fwd_train_validation(lib, case, expect):
    assert fwd_train(lib, **case) == expect


@pytest.mark.parametrize("case,expect", [
    (dict(dq1=None), E_NULL), (dict(dlam=None), E_NULL), (dict(ws=None), E_WS), (dict(ws_bytes=256), E_WS),
    (dict(ws=G[6] + 16), E_ALIGN), (dict(dlam=G[5] + 2), E_ALIGN), (dict(dq1=A[0]), E_ALIAS),
    (dict(dq1=G[1] - 64), E_ALIAS), (dict(dlam=G[6] + 256), E_ALIAS), (dict(ws=A[6] + 1024), E_ALIAS),
    (dict(dtype=F32), E_UNSUP), (dict(B=0), OK), (dict(lh=G[0] + 4), E_ALIAS),
])
def test_bwd_validation(lib, case, expect):
    assert bwd(lib, **case) == expect


def dec_var(lib, T=4, L=100, lens=A[7], out=A[5], ws=A[6], ws_bytes=None, B=2, H=2, d=64, dtype=BF16, lam=0.8):
    if ws_bytes is None:
        ws_bytes = lib.diffattn_decode_varlen_workspace_bytes(B, H, T, L, d)
    return lib.diffattn_decode_varlen(A[0], A[1], A[2], A[3], A[4], out, B, H, T, L, lens, d, dtype, lam, None, 1,
                                      ws, ws_bytes, None)


def split_plan(BH, L, max_keys, min_grid):
    """The decode split plan, restated: at least ceil(L / max_keys) splits per head, more (up to 64 keys per split) to
    reach about min_grid split workgroups, then as many equal splits as the resulting split length needs."""
    s = -(-L // max_keys)
    want, cap = -(-min_grid // BH), -(-L // 64)
    if s < want:
        s = min(want, cap)
    keys = -(-L // s)
    return -(-L // keys)


def merge_groups(splits):
    """States of the merge's first level per item: none up to 32 splits (one pass), else ceil(splits / g) groups of
    g = ceil(sqrt(splits)) splits."""
    if splits <= 32:
        return 0
    g = math.isqrt(splits - 1) + 1
    return -(-splits // g)


@pytest.mark.parametrize("B,H,L", [(64, 16, 8192), (1, 2, 8192), (4, 8, 100000), (2, 3, 777), (128, 16, 65536),
                                   (1, 1, 1 << 20)])
def test_decode_split_plans(lib, B, H, L):
    """One token: splits of at most 4096 keys, more of them (down to 64 keys) to keep ~512 waves; several tokens: at
    most 8192 keys and ~1024 waves (workspace = B H T (splits + first-level groups) x 1040 bytes: m, l and O of both
    maps per state)."""
    for T, max_keys, grid in ((1, 4096, 512), (4, 8192, 1024), (16, 8192, 1024)):
        splits = split_plan(B * H, L, max_keys, grid)
        states = max(splits + merge_groups(splits), ragged_slots(B, H, L))
        assert lib.diffattn_decode_varlen_workspace_bytes(B, H, T, L, 64) == B * H * T * states * 1040, (T, splits)
        if ragged_slots(B, H, L) == 0:   # no balanced plan: a length array changes nothing in the size
            assert lib.diffattn_decode_varlen_workspace_bytes(B, H, T, L, 64) == B * H * T * (
                splits + merge_groups(splits)) * 1040
    # the benchmarked multi-token size: one 8192-key split per head without lengths, 32 balanced slots with them
    assert split_plan(64 * 16, 8192, 8192, 1024) == 1
    assert ragged_slots(64, 16, 8192) == 32


def ragged_slots(B, H, L):
    """States per (head, token) of the balanced plan for ragged caches (0 where the fixed plan serves): at most 512
    sequences, at least 128 (sequence, head) items, keys per wave at least ceil(L / 31) and at most 8192."""
    chunk_min = -(-L // 31)
    if B > 512 or B * H < 128 or chunk_min > 8192:
        return 0
    return (L - 1) // chunk_min + 2


def test_ragged_plan_edges(lib):
    """The balanced plan's eligibility edges in the workspace size: 512 vs 513 sequences, 128 vs 127 items, and the
    longest cache (31 x 8192 rows) whose keys per wave stay within 8192."""
    def ws(B, H, T, L):
        return lib.diffattn_decode_varlen_workspace_bytes(B, H, T, L, 64)
    assert ragged_slots(512, 1, 40) == 21 and ws(512, 1, 1, 40) == 512 * 21 * 1040
    assert ws(513, 1, 1, 40) == 513 * (split_plan(513, 40, 4096, 512)) * 1040
    assert ws(128, 1, 2, 1000) == 128 * 2 * 32 * 1040
    s = split_plan(127, 1000, 8192, 1024)
    assert ws(127, 1, 2, 1000) == 127 * 2 * (s + merge_groups(s)) * 1040
    assert ragged_slots(8, 16, 31 * 8192) == 32 and ragged_slots(8, 16, 31 * 8192 + 1) == 0
    s = split_plan(128, 31 * 8192, 4096, 512)   # 62 splits and 8 groups: more than the balanced plan's 32
    assert ws(8, 16, 1, 31 * 8192) == 128 * max(s + merge_groups(s), 32) * 1040


def test_varlen_workspace_sizes(lib):
    # Without the balanced plan (fewer than 128 heads) the varlen size of one token is the decode's; with it, the
    # larger of the two plans.
    assert (lib.diffattn_decode_varlen_workspace_bytes(1, 16, 1, 8192, 64) ==
            lib.diffattn_decode_workspace_bytes(1, 16, 8192, 64))
    assert (lib.diffattn_decode_varlen_workspace_bytes(64, 16, 1, 8192, 64) ==
            max(lib.diffattn_decode_workspace_bytes(64, 16, 8192, 64), 64 * 16 * 32 * 1040))
    assert lib.diffattn_decode_varlen_workspace_bytes(2, 2, 16, 1000, 64) % (2 * 2 * 16 * 1040) == 0
    for bad in ((2, 2, 0, 100, 64), (2, 2, 17, 100, 64), (2, 2, 8, 7, 64), (2, 2, 4, 100, 8)):
        assert lib.diffattn_decode_varlen_workspace_bytes(*bad) == 0


@pytest.mark.parametrize("case,expect", [
    (dict(T=0), E_SHAPE), (dict(T=17), E_SHAPE), (dict(T=8, L=7), E_SHAPE), (dict(dtype=F32), E_UNSUP),
    (dict(lens=A[7] + 2), E_ALIGN), (dict(lens=A[5]), E_ALIAS), (dict(lens=A[6] + 16), E_ALIAS),
    (dict(ws=None), E_WS), (dict(ws_bytes=64), E_WS), (dict(B=0), OK), (dict(lens=None, out=A[1]), E_ALIAS),
])
def test_decode_varlen_validation(lib, case, expect):
    assert dec_var(lib, **case) == expect


def contiguous_strides(B, H, N):
    out = []
    for w in (64, 64, 64, 64, 128, 128):
        out += [H * N * w, N * w, w]
    return out


def fwd_strided(lib, strides="default", out=A[5], B=1, H=2, N=64, d=64, dtype=BF16, lam=0.5):
    if strides == "default":
        strides = contiguous_strides(B, H, N)
    arr = (ctypes.c_int64 * 18)(*strides) if strides is not None else None
    return lib.diffattn_fwd_strided(A[0], A[1], A[2], A[3], A[4], out, B, H, N, d, dtype, lam, None, 1, 1, arr, None)


def _with(idx, val, B=1, H=2, N=64):
    s = contiguous_strides(B, H, N)
    s[idx] = val
    return s


@pytest.mark.parametrize("case,expect", [
    (dict(strides=None), E_NULL), (dict(strides=_with(2, 68)), E_ALIGN), (dict(strides=_with(14, 64)), E_SHAPE),
    (dict(strides=_with(1, -8)), E_SHAPE), (dict(strides=_with(5, 1 << 26)), E_SHAPE), (dict(out=A[0]), E_ALIAS),
    (dict(dtype=F32), E_UNSUP), (dict(N=0), OK), (dict(strides=_with(11, 64 * 2 * 64 * 4096)), E_SHAPE),
    # outputs that would write one element from several workgroups: the two heads' rows on the same addresses, or
    # overlapping by half a row; both batch entries on the same addresses
    (dict(strides=_with(16, 0)), E_ALIAS), (dict(strides=_with(16, 64)), E_ALIAS),
    (dict(strides=_with(15, 0, B=2), B=2), E_ALIAS),
])
def test_fwd_strided_validation(lib, case, expect):
    assert fwd_strided(lib, **case) == expect


def dec_paged(lib, T=2, max_pages=4, page=16, num_pages=8, table=G[0], lens=G[1], out=A[5], ws=G[2], ws_bytes=None,
              B=2, H=2, d=64, dtype=BF16, lam=0.8, layer=1):
    if ws_bytes is None:
        ws_bytes = lib.diffattn_decode_paged_workspace_bytes(B, H, T, max_pages, page, d)
    return lib.diffattn_decode_paged(A[0], A[1], A[2], A[3], A[4], out, B, H, T, table, max_pages, page, num_pages,
                                     lens, d, dtype, lam, None, layer, ws, ws_bytes, None)


def test_paged_workspace_sizes(lib):
    assert (lib.diffattn_decode_paged_workspace_bytes(4, 8, 3, 20, 64, 64) ==
            lib.diffattn_decode_varlen_workspace_bytes(4, 8, 3, 20 * 64, 64))
    for bad in ((2, 2, 1, 4, 24, 64), (2, 2, 1, 4, 8, 64), (2, 2, 1, 0, 16, 64), (2, 2, 1, 4, 1 << 17, 64),
                (2, 2, 1, 1 << 20, 16, 64), (2, 2, 0, 4, 16, 64), (2, 2, 1, 4, 16, 8)):
        assert lib.diffattn_decode_paged_workspace_bytes(*bad) == 0


@pytest.mark.parametrize("case,expect", [
    (dict(page=24), E_SHAPE), (dict(page=8), E_SHAPE), (dict(page=1 << 17), E_SHAPE), (dict(max_pages=0), E_SHAPE),
    (dict(num_pages=0), E_SHAPE), (dict(T=0), E_SHAPE), (dict(T=17), E_SHAPE),
    (dict(max_pages=1 << 20, ws=None), E_SHAPE), (dict(dtype=F32), E_UNSUP), (dict(d=8), E_UNSUP),
    (dict(table=None), E_NULL), (dict(table=G[0] + 2), E_ALIGN), (dict(lens=G[1] + 2), E_ALIGN),
    (dict(out=G[0]), E_ALIAS), (dict(out=A[1] + 64), E_ALIAS), (dict(out=G[1]), E_ALIAS),
    (dict(ws=None), E_WS), (dict(ws_bytes=64), E_WS), (dict(ws=G[2] + 8), E_ALIGN), (dict(ws=G[0]), E_ALIAS),
    (dict(ws=A[4] + 4096), E_ALIAS), (dict(B=0), OK), (dict(lam=float("nan")), E_LAMBDA), (dict(layer=-1), E_LAYER),
    (dict(lens=None, out=A[3]), E_ALIAS),
])
def test_decode_paged_validation(lib, case, expect):
    assert dec_paged(lib, **case) == expect


# ---------------------------------------------------------------------------------------------------------------
# Strided decode caches: validation only (every case fails before any HIP call, or has no work)
# ---------------------------------------------------------------------------------------------------------------
def token_major(B, H, L, d):
    """Strides of [B][L][H][w] caches viewed as [B][H][L][w]: k1, k2 (w = d) and v (w = 2d)."""
    out = []
    for w in (d, d, 2 * d):
        out += [L * H * w, w, H * w]
    return out


def dec_strided(lib, strides="token", B=2, H=2, T=2, L=64, k1=A[1], k2=A[3], v=A[4], out=A[5], ws=G[2],
                ws_bytes=None, lens=None, d=64, dtype=BF16, lam=0.8, layer=1):
    if isinstance(strides, str):
        strides = token_major(B, H, L, d)
    arr = None if strides is None else (ctypes.c_int64 * 9)(*strides)
    if ws_bytes is None:
        ws_bytes = lib.diffattn_decode_varlen_workspace_bytes(max(B, 0), max(H, 0), max(T, 1), L, 64)
    return lib.diffattn_decode_strided(A[0], k1, A[2], k2, v, out, B, H, T, L, lens, arr, d, dtype, lam, None, layer,
                                       ws, ws_bytes, None)


def with_stride(i, val):
    s = token_major(2, 2, 64, 64)
    s[i] = val
    return s


@pytest.mark.parametrize("case,expect", [
    (dict(strides=None), E_NULL), (dict(strides=None, B=0), OK),
    (dict(strides=with_stride(2, 32)), E_SHAPE),            # k1 row stride below d
    (dict(strides=with_stride(8, 64)), E_SHAPE),            # v row stride below 2d
    (dict(strides=with_stride(0, -8)), E_SHAPE),            # negative batch stride
    (dict(strides=with_stride(1, 4)), E_ALIGN),             # rows not 16-byte aligned
    (dict(strides=with_stride(3, 1 << 62)), E_SHAPE),       # offsets overflow
    (dict(out=A[1] + 2 * 64 * 2 * 64 * 2 - 256), E_ALIAS),  # out ends inside k1's token-major span
    (dict(ws=A[4] + 1024), E_ALIAS),                        # workspace inside v's span
    (dict(dtype=F32), E_UNSUP), (dict(d=8), E_UNSUP), (dict(T=0), E_SHAPE), (dict(T=17), E_SHAPE),
    (dict(layer=-1), E_LAYER), (dict(lam=float("nan")), E_LAMBDA), (dict(lens=G[1] + 2), E_ALIGN),
    # K1, K2 and V packed in one buffer may overlap each other: validation reaches the workspace check.
    (dict(k2=A[1] + 128, v=A[1] + 256, strides=[64 * 2 * 256, 256, 2 * 256] * 3, ws=None), E_WS),
])
def test_decode_strided_validation(lib, case, expect):
    assert dec_strided(lib, **case) == expect


# Strided training: a packed projection [B][N][H][6][64] (q1 | k1 | q2 | k2 | v) at A[0] and its packed gradient
# buffer at G[0]; dy dense at A[7].  Every case changes the default (which itself would pass validation and is never
# called) so that validation fails.
def packed_strides(B, H, N, col, w):
    del w
    return [N * H * 384, 384, H * 384], col


def train_strided_layout(B=1, H=2, N=64):
    s_in, s_g = [], []
    ptr_in, ptr_g = [], []
    for col, w in ((0, 64), (64, 64), (128, 64), (192, 64), (256, 128)):
        st, c = packed_strides(B, H, N, col, w)
        s_in += st
        ptr_in.append(A[0] + 2 * c)
        s_g += st
        ptr_g.append(G[0] + 2 * c)
    dy = [H * N * 128, N * 128, 128]
    return ptr_in, ptr_g, s_in, dy, s_g


def bwd_strided(lib, edit=None, ptr_edit=None, B=1, H=2, N=64, dtype=BF16, strides_none=False):
    ptr_in, ptr_g, s_in, s_dy, s_g = train_strided_layout(B, H, N)
    strides = s_in + s_dy + s_g
    ptrs = ptr_in + [A[7]] + ptr_g
    if edit:
        for i, v in edit.items():
            strides[i] = v
    if ptr_edit:
        for i, v in ptr_edit.items():
            ptrs[i] = v
    arr = None if strides_none else (ctypes.c_int64 * 33)(*strides)
    ws_bytes = lib.diffattn_bwd_workspace_bytes(B, H, N, 64)
    return lib.diffattn_bwd_strided(*ptrs[:6], A[6], *ptrs[6:], G[5], B, H, N, 64, dtype, 0.5, None, 1, 1, arr,
                                    G[6], ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    (dict(strides_none=True), E_NULL),
    (dict(edit={2: 772}), E_ALIGN),                        # q1 row stride not a multiple of 8
    (dict(edit={14: 120}), E_SHAPE),                       # v row stride below its 128-element row
    (dict(edit={4: -384}), E_SHAPE),                       # negative head stride
    (dict(edit={5: 1 << 24}), E_SHAPE),                    # k1's N + 256 rows past 4 GiB of buffer offsets
    (dict(ptr_edit={6: A[0]}), E_ALIAS),                   # dq1 written over q1
    (dict(ptr_edit={7: G[0] + 64}), E_ALIAS),              # dk1 overlapping dq1 inside each packed row
    (dict(ptr_edit={10: G[0] + 2 * 320}), E_ALIAS),        # dv (128 wide) running into the next head's dq1
    (dict(ptr_edit={5: G[0] + 2 * 64}), E_ALIAS),          # dy read from where dk1 is written
    (dict(edit={19: 0}), E_ALIAS),                         # dq1 of both heads on the same addresses
    (dict(edit={31: 64}), E_ALIAS),                        # dv heads 64 elements apart, rows 128 wide
    # dq1 alone in a buffer of its own, dense 64-element rows, but head 1 starting at head 0's row 32 (N = 64)
    (dict(ptr_edit={6: 0x900000000}, edit={20: 64, 19: 32 * 64}), E_ALIAS),
    (dict(dtype=F32), E_UNSUP), (dict(B=0), OK),
])
def test_bwd_strided_validation(lib, case, expect):
    assert bwd_strided(lib, **case) == expect


def fwd_train_strided(lib, strides_none=False, out=None, saved=A[6], edit=None, N=64):
    ptr_in, _, s_in, _, _ = train_strided_layout(N=N)
    s = s_in + [2 * N * 128, N * 128, 128]
    if edit:
        for i, v in edit.items():
            s[i] = v
    arr = None if strides_none else (ctypes.c_int64 * 18)(*s)
    need = lib.diffattn_train_saved_bytes(1, 2, N, 64)
    return lib.diffattn_fwd_train_strided(*ptr_in, A[5] if out is None else out, 1, 2, N, 64, BF16, 0.5, None, 1, 1,
                                          arr, saved, need, None)


@pytest.mark.parametrize("case,expect", [
    (dict(strides_none=True), E_NULL), (dict(out=A[0] + 2 * 64), E_ALIAS), (dict(saved=A[0]), E_ALIAS),
    (dict(saved=A[6] + 8), E_ALIGN), (dict(edit={17: 64}), E_SHAPE), (dict(N=0), OK),
    (dict(edit={16: 0}), E_ALIAS), (dict(edit={16: 64}), E_ALIAS),   # out heads folded onto each other
])
def test_fwd_train_strided_validation(lib, case, expect):
    assert fwd_train_strided(lib, **case) == expect


def test_decode_noalloc_rejects_oversized_partials(lib):
    """Partials beyond the library's scratch array are DIFFATTN_ERR_WORKSPACE before any HIP call; shape errors are
    reported as for diffattn_decode."""
    B, H, L = 64, 16, 65536   # 16 splits of 4096 keys per head: 17.0 MB of partials
    assert lib.diffattn_decode_workspace_bytes(B, H, L, 64) > da.NOALLOC_SCRATCH_BYTES
    assert lib.diffattn_decode_workspace_bytes(B, H, 61440, 64) <= da.NOALLOC_SCRATCH_BYTES
    assert lib.diffattn_decode_noalloc(A[0], A[1], A[2], A[3], A[4], A[5], B, H, L, 64, BF16, 0.8, 1, 1,
                                       None) == E_WS
    assert lib.diffattn_decode_noalloc(A[0], A[1], A[2], A[3], A[4], A[5], 1, 1, 0, 64, BF16, 0.8, 1, 1,
                                       None) == E_SHAPE
    assert lib.diffattn_decode_noalloc(A[0], A[1], A[2], A[3], A[4], A[5], 1, 1, 64, 32, BF16, 0.8, 1, 1,
                                       None) == E_UNSUP
