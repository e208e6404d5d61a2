"""CPU checks of the C ABI: the library loads, exports every function that
include/zg_attn.h declares, sizes workspaces as documented and rejects bad
arguments before launching anything (host-side failure handling; no kernel
runs in these tests)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zg_attn.h")


@pytest.fixture(scope="module")
def bd():
    from global_attention_zg_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("zg_attn_fwd", "zg_attn_decode", "zg_attn_fwd_workspace_size",
              "zg_attn_decode_workspace_size", "zg_attn_decode_num_splits", "zg_attn_strerror",
              "zg_attn_decode_paged", "zg_attn_kv_write_pages", "zg_attn_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol(bd):
    lib = ctypes.CDLL(bd.library_path())
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(bd.EXPORTED)


def test_strerror(bd):
    assert bd.zg_attn_strerror(0) == "ok"
    for st in (-1, -2, -3, -4, -5):
        assert bd.zg_attn_strerror(st) and bd.zg_attn_strerror(st) != "unknown status"
    assert bd.zg_attn_strerror(-99) == "unknown status"


def _fwd(bd, p, **ptrs):
    names = ["q", "k", "v", "gate", "qw", "kw", "out", "lse", "kout", "ws"]
    args = [ptrs.get(n) for n in names]
    return bd._lib.zg_attn_fwd(ctypes.byref(p), *args[:10], ptrs.get("ws_bytes", 0), None)


FAKE = 0x10000000  # 16-byte aligned, never dereferenced: validation fails first


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, -2), ("head_dim", 0, -1), ("n_kv_heads", 3, -1), ("n_q_heads", 0, -1),
    ("rope_dim", 43, -1), ("rope_dim", 66, -2), ("rope_dim", 130, -1), ("window", -1, -1),
    ("batch", -1, -1), ("seqlen", -5, -1), ("rms_eps", -1.0, -1), ("softmax_scale", -0.5, -1),
    ("rope_theta", 0.0, -1), ("rms_eps", float("nan"), -1),
])
def test_fwd_rejects_bad_params(bd, field, value, status):
    p = bd.make_params(1, 64, 32, 8, 128, 128)
    setattr(p, field, value)
    assert _fwd(bd, p, q=FAKE, k=FAKE, v=FAKE, qw=FAKE, kw=FAKE, out=FAKE, ws=FAKE,
                ws_bytes=1 << 30) == status
    assert bd.zg_attn_fwd_workspace_size(p) == 0


def test_fwd_group_size_support(bd):
    p = bd.make_params(1, 64, 24, 8, 128, 128)   # group of 3
    assert _fwd(bd, p) == bd.ZG_ERR_UNSUPPORTED
    p = bd.make_params(1, 64, 32, 2, 128, 128)   # group of 16
    assert _fwd(bd, p) == bd.ZG_ERR_UNSUPPORTED


def test_fwd_null_and_misaligned_pointers(bd):
    p = bd.make_params(1, 64, 32, 8, 128, 128)
    ok = dict(q=FAKE, k=FAKE, v=FAKE, qw=FAKE, kw=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    for name in ("q", "k", "v", "qw", "kw", "out"):
        a = dict(ok)
        a[name] = None
        assert _fwd(bd, p, **a) == bd.ZG_ERR_INVALID, name
        a[name] = FAKE + 2
        assert _fwd(bd, p, **a) == bd.ZG_ERR_INVALID, name
    a = dict(ok, gate=FAKE + 8)
    assert _fwd(bd, p, **a) == bd.ZG_ERR_INVALID
    a = dict(ok, lse=FAKE + 2)
    assert _fwd(bd, p, **a) == bd.ZG_ERR_INVALID


def test_fwd_workspace_rules(bd):
    p = bd.make_params(2, 100, 32, 8, 128, 128)
    need = bd.zg_attn_fwd_workspace_size(p)
    assert need == 2 * 100 * 8 * 128 * 2
    base = dict(q=FAKE, k=FAKE, v=FAKE, qw=FAKE, kw=FAKE, out=FAKE)
    assert _fwd(bd, p, **base) == bd.ZG_ERR_WORKSPACE
    assert _fwd(bd, p, **dict(base, ws=FAKE, ws_bytes=need - 1)) == bd.ZG_ERR_WORKSPACE
    assert _fwd(bd, p, **dict(base, ws=FAKE + 8, ws_bytes=need)) == bd.ZG_ERR_INVALID


def test_fwd_global_workspace_holds_queue_counters(bd):
    """A global layer (window 0) keeps the causal kernel's 256 bytes of
    work-queue counters after K' in its workspace, and needs them also when
    K' goes to k_out."""
    p = bd.make_params(2, 100, 32, 8, 128, 0)
    need = bd.zg_attn_fwd_workspace_size(p)
    assert need == 2 * 100 * 8 * 128 * 2 + bd.QUEUE_BYTES == 409856
    base = dict(q=FAKE, k=FAKE, v=FAKE, qw=FAKE, kw=FAKE, out=FAKE)
    assert _fwd(bd, p, **dict(base, ws=FAKE, ws_bytes=need - 1)) == bd.ZG_ERR_WORKSPACE
    assert _fwd(bd, p, **dict(base, kout=FAKE)) == bd.ZG_ERR_WORKSPACE
    assert _fwd(bd, p, **dict(base, kout=FAKE, ws=FAKE, ws_bytes=255)) == bd.ZG_ERR_WORKSPACE
    assert _fwd(bd, p, **dict(base, kout=FAKE, ws=FAKE + 8, ws_bytes=256)) == bd.ZG_ERR_INVALID
    # K' rows not a multiple of 256 bytes apart: the counters start on the next 256
    assert bd.zg_attn_fwd_fp8_workspace_size(bd.make_params(1, 3, 4, 1, 128, 0)) == 512 + 256
    assert bd.zg_attn_fwd_fp8_workspace_size(bd.make_params(1, 2, 4, 1, 128, 0)) == 256 + 256
    assert bd.zg_attn_fwd_fp8_workspace_size(bd.make_params(1, 4, 4, 1, 128, 0)) == 512 + 256
    assert bd.zg_attn_fwd_varlen_workspace_size(p, 5000) == 5000 * 8 * 128 * 2 + 256
    assert bd.zg_attn_fwd_varlen_workspace_size(p, 0) == 0
    for B, S in ((0, 64), (1, 0)):
        assert bd.zg_attn_fwd_workspace_size(bd.make_params(B, S, 32, 8, 128, 0)) == 0


def test_fwd_empty_launches_nothing(bd):
    for B, S in ((0, 64), (1, 0), (0, 0)):
        p = bd.make_params(B, S, 32, 8, 128, 128)
        assert _fwd(bd, p) == bd.ZG_OK
        assert bd.zg_attn_fwd_workspace_size(p) == 0


def _dec(bd, p, cap, ring, num_splits=0, **ptrs):
    names = ["q", "kn", "vn", "kc", "vc", "sl"]
    a = [ptrs.get(n) for n in names]
    return bd._lib.zg_attn_decode(ctypes.byref(p), *a, cap, ring, ptrs.get("gate"),
                                  ptrs.get("qw"), ptrs.get("kw"), ptrs.get("out"), num_splits,
                                  ptrs.get("ws"), ptrs.get("ws_bytes", 0), None)


def test_decode_splits_and_workspace(bd):
    p = bd.make_params(16, 0, 32, 8, 128, 0)
    ns = bd.zg_attn_decode_num_splits(p, 262145)
    assert 1 <= ns <= 64
    assert bd.zg_attn_decode_workspace_size(p, 262145, 0) == 16 * 32 * ns * 130 * 4
    assert bd.zg_attn_decode_workspace_size(p, 262145, 5) == 16 * 32 * 5 * 130 * 4
    p2 = bd.make_params(16, 0, 32, 8, 128, 128)
    assert bd.zg_attn_decode_num_splits(p2, 128) == 1
    assert bd.zg_attn_decode_workspace_size(p, 0, 0) == 0
    assert bd.zg_attn_decode_workspace_size(p, 100, 300) == 0


def test_decode_rejects_bad_arguments(bd):
    ok = dict(q=FAKE, kc=FAKE, vc=FAKE, sl=FAKE, qw=FAKE, kw=FAKE, out=FAKE, ws=FAKE,
              ws_bytes=1 << 30)
    p = bd.make_params(2, 0, 32, 8, 128, 128)
    assert _dec(bd, p, 128, 1, **dict(ok, kn=FAKE)) == bd.ZG_ERR_INVALID      # k without v
    assert _dec(bd, p, 64, 1, **ok) == bd.ZG_ERR_INVALID                      # window != cap
    assert _dec(bd, p, 0, 0, **ok) == bd.ZG_ERR_INVALID
    assert _dec(bd, p, 128, 2, **ok) == bd.ZG_ERR_INVALID
    assert _dec(bd, p, 128, 1, num_splits=257, **ok) == bd.ZG_ERR_INVALID
    assert _dec(bd, p, 128, 1, **dict(ok, sl=None)) == bd.ZG_ERR_INVALID
    assert _dec(bd, p, 128, 1, **dict(ok, sl=FAKE + 2)) == bd.ZG_ERR_INVALID
    assert _dec(bd, p, 128, 1, **dict(ok, ws=None)) == bd.ZG_ERR_WORKSPACE
    assert _dec(bd, p, 128, 1, **dict(ok, ws_bytes=16)) == bd.ZG_ERR_WORKSPACE
    p0 = bd.make_params(0, 0, 32, 8, 128, 128)
    assert _dec(bd, p0, 128, 1) == bd.ZG_OK
    pbad = bd.make_params(2, 0, 32, 8, 96, 128)
    assert _dec(bd, pbad, 128, 1, **ok) == bd.ZG_ERR_UNSUPPORTED


def _dec_noalloc(bd, p, cap, ring, num_splits=0, **ptrs):
    a = [ptrs.get(n) for n in ("q", "kn", "vn", "kc", "vc", "sl")]
    return bd._lib.zg_attn_decode_noalloc(ctypes.byref(p), *a, cap, ring, ptrs.get("gate"),
                                          ptrs.get("qw"), ptrs.get("kw"), ptrs.get("out"),
                                          num_splits, None)


def test_noalloc_decode_rejects_before_any_hip_call(bd):
    """Every rejection, the size limit included, comes before the library
    touches HIP (the scratch address lookup), so it holds on a host without a
    GPU."""
    ok = dict(q=FAKE, kc=FAKE, vc=FAKE, sl=FAKE, qw=FAKE, kw=FAKE, out=FAKE)
    p = bd.make_params(2, 0, 32, 8, 128, 0)
    assert _dec_noalloc(bd, p, 128, 2, **ok) == bd.ZG_ERR_INVALID
    assert _dec_noalloc(bd, p, 0, 0, **ok) == bd.ZG_ERR_INVALID
    assert _dec_noalloc(bd, p, 128, 0, num_splits=257, **ok) == bd.ZG_ERR_INVALID
    assert _dec_noalloc(bd, bd.make_params(2, 0, 32, 8, 96, 0), 128, 0, **ok) == bd.ZG_ERR_UNSUPPORTED
    assert _dec_noalloc(bd, bd.make_params(0, 0, 32, 8, 128, 0), 128, 0) == bd.ZG_OK
    # the partials of 64 sequences x 32 heads x 64 splits (68 MB) exceed the array
    big = bd.make_params(64, 0, 32, 8, 128, 0)
    need = bd.zg_attn_decode_workspace_size(big, 1 << 20, 64)
    assert need > (8 << 20)
    assert _dec_noalloc(bd, big, 1 << 20, 0, num_splits=64, **ok) == bd.ZG_ERR_TOO_LARGE
    assert "scratch" in bd.zg_attn_strerror(bd.ZG_ERR_TOO_LARGE)


def _dec_fp8(bd, p, cap, ring, k_scale, v_scale, num_splits=0, **ptrs):
    a = [ptrs.get(n) for n in ("q", "kn", "vn", "kc", "vc", "sl")]
    return bd._lib.zg_attn_decode_fp8(ctypes.byref(p), *a, cap, ring, k_scale, v_scale,
                                      ptrs.get("gate"), ptrs.get("qw"), ptrs.get("kw"),
                                      ptrs.get("out"), num_splits, ptrs.get("ws"),
                                      ptrs.get("ws_bytes", 0), None)


def _dec_paged_fp8(bd, p, num_pages, max_pages, page_size, k_scale, v_scale, **ptrs):
    a = [ptrs.get(n) for n in ("q", "kn", "vn", "kp", "vp")]
    return bd._lib.zg_attn_decode_paged_fp8(ctypes.byref(p), *a, num_pages, ptrs.get("bt"),
                                            max_pages, page_size, ptrs.get("sl"), k_scale,
                                            v_scale, ptrs.get("gate"), ptrs.get("qw"),
                                            ptrs.get("kw"), ptrs.get("out"), 0, ptrs.get("ws"),
                                            ptrs.get("ws_bytes", 0), None)


def test_fp8_decode_rejects_bad_arguments(bd):
    """Every case fails validation, so nothing is launched."""
    ok = dict(q=FAKE, kc=FAKE, vc=FAKE, sl=FAKE, qw=FAKE, kw=FAKE, out=FAKE, ws=FAKE,
              ws_bytes=1 << 30)
    p = bd.make_params(2, 0, 32, 8, 128, 128)
    inf, nan = float("inf"), float("nan")
    for ks, vs in ((0.0, 1.0), (1.0, 0.0), (-1.0, 1.0), (1.0, -3.0), (inf, 1.0), (1.0, nan)):
        assert _dec_fp8(bd, p, 128, 1, ks, vs, **ok) == bd.ZG_ERR_INVALID, (ks, vs)
    assert _dec_fp8(bd, p, 64, 1, 1.0, 1.0, **ok) == bd.ZG_ERR_INVALID         # window != cap
    assert _dec_fp8(bd, p, 128, 1, 1.0, 1.0, **dict(ok, kn=FAKE)) == bd.ZG_ERR_INVALID
    assert _dec_fp8(bd, p, 128, 1, 1.0, 1.0, **dict(ok, kc=FAKE + 8)) == bd.ZG_ERR_INVALID
    assert _dec_fp8(bd, p, 128, 1, 1.0, 1.0, **dict(ok, ws_bytes=16)) == bd.ZG_ERR_WORKSPACE
    p0 = bd.make_params(0, 0, 32, 8, 128, 128)
    assert _dec_fp8(bd, p0, 128, 1, 1.0, 1.0) == bd.ZG_OK
    okp = dict(q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, qw=FAKE, kw=FAKE, out=FAKE, ws=FAKE,
               ws_bytes=1 << 30)
    pg = bd.make_params(2, 0, 32, 8, 128, 0)
    assert _dec_paged_fp8(bd, pg, 8, 4, 64, 0.0, 1.0, **okp) == bd.ZG_ERR_INVALID
    assert _dec_paged_fp8(bd, pg, 8, 4, 48, 1.0, 1.0, **okp) == bd.ZG_ERR_INVALID
    assert _dec_paged_fp8(bd, pg, 8, 4, 64, 1.0, 1.0, **dict(okp, bt=None)) == bd.ZG_ERR_INVALID


def _bwd(bd, p, **ptrs):
    names = ["q", "k", "v", "gate", "qw", "kw", "out", "lse", "dout", "dq", "dk", "dv", "dgate",
             "dqw", "dkw", "ws"]
    args = [ptrs.get(n) for n in names]
    return bd._lib.zg_attn_bwd(ctypes.byref(p), *args, ptrs.get("ws_bytes", 0), None)


@pytest.mark.parametrize("window", [128, 0, 300, 299])
def test_bwd_workspace_size_formula(bd, window):
    B, S, Hq, Hkv, D = 2, 300, 32, 8, 128
    p = bd.make_params(B, S, Hq, Hkv, D, window)
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    spad = (S + 127) // 128 * 128
    grp = Hq // Hkv
    hpw = min(grp, 4)                                     # query heads per dq' workgroup
    n_dq = -(-S // (128 // hpw)) * B * Hkv * (grp // hpw)  # dq' workgroups
    n_dkv = -(-S // 128) * B * Hkv                         # dk'/dv workgroups
    want = (a(B * S * Hq * D * 2) + a(B * S * Hkv * D * 2) + a(B * S * Hq * D * 2)
            + 2 * a(B * Hq * spad * 4) + a(n_dq * D * 4) + a(n_dkv * D * 4)
            + a(2 * 256 * D * 4))
    assert bd.zg_attn_bwd_workspace_size(p) == want
    p.head_dim = 64
    assert bd.zg_attn_bwd_workspace_size(p) == 0


def test_bwd_rejects_bad_arguments(bd):
    p = bd.make_params(1, 64, 32, 8, 128, 128)
    full = dict(q=FAKE, k=FAKE, v=FAKE, qw=FAKE, kw=FAKE, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE,
                dk=FAKE, dv=FAKE, dqw=FAKE, dkw=FAKE, ws=FAKE, ws_bytes=1 << 40)
    for missing in ("q", "out", "lse", "dout", "dq", "dk", "dv", "dqw", "dkw"):
        args = dict(full)
        args[missing] = None
        assert _bwd(bd, p, **args) == bd.ZG_ERR_INVALID, missing
    # gate and dgate come together
    assert _bwd(bd, p, **dict(full, gate=FAKE)) == bd.ZG_ERR_INVALID
    assert _bwd(bd, p, **dict(full, dgate=FAKE)) == bd.ZG_ERR_INVALID
    # misaligned tensor
    assert _bwd(bd, p, **dict(full, dq=FAKE + 8)) == bd.ZG_ERR_INVALID
    # workspace missing or short
    assert _bwd(bd, p, **dict(full, ws=None)) == bd.ZG_ERR_WORKSPACE
    need = bd.zg_attn_bwd_workspace_size(p)
    assert _bwd(bd, p, **dict(full, ws_bytes=need - 1)) == bd.ZG_ERR_WORKSPACE
    # bad params are checked first
    p.rope_dim = 43
    assert _bwd(bd, p, **full) == bd.ZG_ERR_INVALID
    # empty problem: valid, nothing launched
    q = bd.make_params(0, 64, 32, 8, 128, 0)
    assert _bwd(bd, q) == bd.ZG_OK


def _dec_paged(bd, p, num_pages, max_pages, page_size, num_splits=0, **ptrs):
    a = [ptrs.get(n) for n in ("q", "kn", "vn", "kp", "vp")]
    return bd._lib.zg_attn_decode_paged(ctypes.byref(p), *a, num_pages, ptrs.get("bt"),
                                        max_pages, page_size, ptrs.get("sl"), ptrs.get("gate"),
                                        ptrs.get("qw"), ptrs.get("kw"), ptrs.get("out"),
                                        num_splits, ptrs.get("ws"), ptrs.get("ws_bytes", 0), None)


def _write_pages(bd, p, num_pages, max_pages, page_size, **ptrs):
    a = [ptrs.get(n) for n in ("kp_in", "v_in", "kp", "vp")]
    return bd._lib.zg_attn_kv_write_pages(ctypes.byref(p), *a, num_pages, ptrs.get("bt"),
                                          max_pages, page_size, None)


def test_paged_decode_rejects_bad_arguments(bd):
    ok = dict(q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, qw=FAKE, kw=FAKE, out=FAKE, ws=FAKE,
              ws_bytes=1 << 30)
    p = bd.make_params(2, 0, 32, 8, 128, 0)
    for page_size in (16, 48, 100, 1 << 17):                       # not a power of two in range
        assert _dec_paged(bd, p, 8, 4, page_size, **ok) == bd.ZG_ERR_INVALID, page_size
    assert _dec_paged(bd, p, 0, 4, 64, **ok) == bd.ZG_ERR_INVALID  # empty pool
    assert _dec_paged(bd, p, 8, 0, 64, **ok) == bd.ZG_ERR_INVALID  # empty table row
    assert _dec_paged(bd, p, 8, 1 << 16, 1 << 16, **ok) == bd.ZG_ERR_INVALID  # > int slots
    assert _dec_paged(bd, p, 8, 4, 64, **dict(ok, bt=None)) == bd.ZG_ERR_INVALID
    assert _dec_paged(bd, p, 8, 4, 64, **dict(ok, bt=FAKE + 2)) == bd.ZG_ERR_INVALID
    assert _dec_paged(bd, p, 8, 4, 64, **dict(ok, kp=FAKE + 8)) == bd.ZG_ERR_INVALID
    assert _dec_paged(bd, p, 8, 4, 64, **dict(ok, kn=FAKE)) == bd.ZG_ERR_INVALID  # k without v
    assert _dec_paged(bd, p, 8, 4, 64, num_splits=257, **ok) == bd.ZG_ERR_INVALID
    # workspace sized for cap = max_pages * page_size
    need = bd.zg_attn_decode_workspace_size(p, 4 * 64, 0)
    assert _dec_paged(bd, p, 8, 4, 64, **dict(ok, ws_bytes=need - 1)) == bd.ZG_ERR_WORKSPACE
    p0 = bd.make_params(0, 0, 32, 8, 128, 0)
    assert _dec_paged(bd, p0, 8, 4, 64, bt=FAKE) == bd.ZG_OK
    pbad = bd.make_params(2, 0, 32, 8, 128, 0)
    pbad.rope_dim = 43
    assert _dec_paged(bd, pbad, 8, 4, 64, **ok) == bd.ZG_ERR_INVALID


def test_write_pages_rejects_bad_arguments(bd):
    ok = dict(kp_in=FAKE, v_in=FAKE, kp=FAKE, vp=FAKE, bt=FAKE)
    p = bd.make_params(2, 300, 8, 8, 128)
    assert _write_pages(bd, p, 16, 9, 32, **ok) == bd.ZG_ERR_INVALID     # 288 slots < 300
    assert _write_pages(bd, p, 16, 10, 24, **ok) == bd.ZG_ERR_INVALID
    assert _write_pages(bd, p, 16, 10, 32, **dict(ok, v_in=None)) == bd.ZG_ERR_INVALID
    assert _write_pages(bd, p, 16, 10, 32, **dict(ok, vp=FAKE + 4)) == bd.ZG_ERR_INVALID
    assert _write_pages(bd, p, 0, 10, 32, **ok) == bd.ZG_ERR_INVALID
    for B, S in ((0, 300), (2, 0)):
        assert _write_pages(bd, bd.make_params(B, S, 8, 8, 128), 16, 10, 32, bt=FAKE) == bd.ZG_OK


def _fwd_varlen(bd, p, total, **ptrs):
    names = ["q", "k", "v", "gate", "qw", "kw", "out", "lse", "kout", "ws"]
    args = [ptrs.get(n) for n in names]
    return bd._lib.zg_attn_fwd_varlen(ctypes.byref(p), ptrs.get("cu"), total, *args,
                                      ptrs.get("ws_bytes", 0), None)


def test_fwd_varlen_workspace_and_rejects(bd):
    p = bd.make_params(3, 4096, 32, 8, 128, 128)
    assert bd.zg_attn_fwd_varlen_workspace_size(p, 5000) == 5000 * 8 * 128 * 2
    assert bd.zg_attn_fwd_varlen_workspace_size(p, -1) == 0
    full = dict(cu=FAKE, q=FAKE, k=FAKE, v=FAKE, qw=FAKE, kw=FAKE, out=FAKE, ws=FAKE,
                ws_bytes=5000 * 8 * 128 * 2)
    assert _fwd_varlen(bd, p, 5000, **dict(full, cu=None)) == bd.ZG_ERR_INVALID
    assert _fwd_varlen(bd, p, 5000, **dict(full, cu=FAKE + 2)) == bd.ZG_ERR_INVALID
    assert _fwd_varlen(bd, p, -5, **full) == bd.ZG_ERR_INVALID
    assert _fwd_varlen(bd, p, 5000, **dict(full, k=None)) == bd.ZG_ERR_INVALID
    assert _fwd_varlen(bd, p, 5000, **dict(full, out=FAKE + 8)) == bd.ZG_ERR_INVALID
    assert _fwd_varlen(bd, p, 5000, **dict(full, ws_bytes=5000 * 8 * 128 * 2 - 1)) == \
        bd.ZG_ERR_WORKSPACE
    # empty batch, empty grid or no tokens: valid, nothing launched
    assert _fwd_varlen(bd, bd.make_params(0, 4096, 32, 8, 128, 0), 0) == bd.ZG_OK
    assert _fwd_varlen(bd, bd.make_params(3, 0, 32, 8, 128, 0), 0, cu=FAKE) == bd.ZG_OK
    assert _fwd_varlen(bd, p, 0, cu=FAKE) == bd.ZG_OK
    p.n_kv_heads = 3
    assert _fwd_varlen(bd, p, 5000, **full) == bd.ZG_ERR_INVALID


def test_projection_argument_rules(bd):
    lin = bd._lib.zg_linear
    assert lin(0, 256, 64, None, None, None, None) == bd.ZG_OK          # nothing to do
    assert lin(5, 0, 64, None, None, None, None) == bd.ZG_OK
    assert lin(-1, 256, 64, FAKE, FAKE, FAKE, None) == bd.ZG_ERR_INVALID
    assert lin(5, 200, 64, FAKE, FAKE, FAKE, None) == bd.ZG_ERR_UNSUPPORTED  # N % 256
    assert lin(5, 256, 48, FAKE, FAKE, FAKE, None) == bd.ZG_ERR_UNSUPPORTED  # K % 32
    assert lin(5, 256, 64, None, FAKE, FAKE, None) == bd.ZG_ERR_INVALID
    assert lin(5, 256, 64, FAKE, FAKE, FAKE + 8, None) == bd.ZG_ERR_INVALID
    proj = bd._lib.zg_qkvg_proj
    p = bd.make_params(2, 100, 32, 8, 128)
    args = [FAKE] * 5
    assert proj(ctypes.byref(p), 4096, None, *args[1:], None, None) == bd.ZG_ERR_INVALID
    assert proj(ctypes.byref(p), 4010, *args, None, None) == bd.ZG_ERR_UNSUPPORTED  # hidden % 32
    assert proj(ctypes.byref(p), 4096, *args[:4], None, None, None) == bd.ZG_ERR_INVALID  # no v
    assert proj(ctypes.byref(p), 4096, *args, FAKE + 4, None) == bd.ZG_ERR_INVALID  # gate
    p1 = bd.make_params(2, 100, 4, 1, 128)   # Hkv * D = 128: not a whole 256-column tile
    assert proj(ctypes.byref(p1), 4096, *args, None, None) == bd.ZG_ERR_UNSUPPORTED
    p0 = bd.make_params(0, 100, 32, 8, 128)
    assert proj(ctypes.byref(p0), 4096, None, None, None, None, None, None, None) == bd.ZG_OK


def test_fp8_argument_rules(bd):
    qz = bd._lib.zg_quantize_fp8
    assert qz(0, None, 1.0, None, None) == bd.ZG_OK
    assert qz(-8, FAKE, 1.0, FAKE, None) == bd.ZG_ERR_INVALID
    assert qz(8, FAKE, 0.0, FAKE, None) == bd.ZG_ERR_INVALID          # scale must be > 0
    assert qz(8, FAKE, float("inf"), FAKE, None) == bd.ZG_ERR_INVALID
    assert qz(12, FAKE, 1.0, FAKE, None) == bd.ZG_ERR_UNSUPPORTED     # n % 8
    assert qz(8, FAKE + 8, 1.0, FAKE, None) == bd.ZG_ERR_INVALID      # x alignment
    assert qz(8, FAKE, 1.0, FAKE + 4, None) == bd.ZG_ERR_INVALID      # q alignment
    lf = bd._lib.zg_linear_fp8
    assert lf(0, 256, 128, None, None, 1.0, None, None) == bd.ZG_OK
    assert lf(5, 256, 64, FAKE, FAKE, 1.0, FAKE, None) == bd.ZG_ERR_UNSUPPORTED   # K % 128
    assert lf(5, 100, 128, FAKE, FAKE, 1.0, FAKE, None) == bd.ZG_ERR_UNSUPPORTED  # N % 256
    assert lf(5, 256, 128, FAKE, None, 1.0, FAKE, None) == bd.ZG_ERR_INVALID
    assert lf(5, 256, 128, FAKE, FAKE, float("nan"), FAKE, None) == bd.ZG_ERR_INVALID
