"""The C-ABI library on a host without a GPU: it loads, exports every entry point
include/gdn.h declares, and its host-side validation rejects bad arguments before
anything is launched (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from linear_attention_chunked_gdn_amd import build, gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.LIB_PATH):
        build.build_library()
    return gdn.load_library()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["gdn_prefill", "gdn_decode_step", "gdn_prefill_plan", "gdn_status_string", "gdn_last_error",
         "gdn_kda_workspace_size", "gdn_kda_prefill", "gdn_kda_decode_step", "gdn_prefill_fused",
         "gdn_decode_step_fused", "gdn_prefill_split", "gdn_prefill_split_workspace_size",
         "gdn_prefill_seg", "gdn_prefill_seg_workspace_size", "gdn_prefill_seg_choose",
         "gdn_prefill_split_fused", "gdn_kda_prefill_seg", "gdn_prefill_split_noalloc",
         "gdn_prefill_auto_plan", "gdn_prefill_auto"])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", build.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdn_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, f"{name} is declared in gdn.h but not exported"
        assert hasattr(lib, name)


def test_header_compiles_as_c():
    src = f'#include "{HEADER}"\nint main(void) {{ return (int)GDN_OK; }}\n'
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-x", "c", "-", "-o", os.devnull],
                         input=src, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_status_strings(lib):
    assert lib.gdn_status_string(0) == b"ok"
    assert lib.gdn_status_string(1) == b"invalid argument"
    assert lib.gdn_status_string(2) == b"unsupported"
    assert lib.gdn_status_string(3) == b"device error"


def _prefill(lib, **over):
    # fake, 16-byte aligned, never-dereferenced addresses: validation fails before any use
    a = dict(q=0x10000, k=0x20000, v=0x30000, g=0x40000, beta=0x50000, s0=None, cu=None,
             N=1, T=10, Hk=2, Hv=4, Dk=128, Dv=128, C=64, io=1, o=0x60000, fs=None)
    a.update(over)
    p = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lib.gdn_prefill(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["s0"]),
                           p(a["cu"]), a["N"], a["T"], a["Hk"], a["Hv"], a["Dk"], a["Dv"], a["C"],
                           a["io"], p(a["o"]), p(a["fs"]), None)


@pytest.mark.parametrize("over,status,msg", [
    (dict(Hv=3), 1, "multiple"),
    (dict(Dk=64), 2, "Dk=64"),
    (dict(Dv=256), 2, "Dv=256"),
    (dict(C=32), 2, "chunk_size"),
    (dict(N=0), 1, "N=0"),
    (dict(T=-1), 1, "T_tot"),
    (dict(N=2), 1, "cu_seqlens"),
    (dict(q=None), 1, "non-null"),
    (dict(io=7), 1, "io_dtype"),
    (dict(io=3), 1, "io_dtype"),
    (dict(io=2, k=0x20008), 1, "aligned"),
    (dict(k=0x20008), 1, "aligned"),
    (dict(o=0x30000), 1, "overlaps"),
    (dict(s0=0x70000, fs=0x70100), 1, "final_state overlaps"),
])
def test_prefill_rejects(lib, over, status, msg):
    st = _prefill(lib, **over)
    assert st == status
    assert msg in lib.gdn_last_error().decode()


def test_prefill_nothing_to_do_is_ok(lib):
    # T_tot = 0 without a final state: valid, and nothing is launched
    assert _prefill(lib, q=None, k=None, v=None, g=None, beta=None, o=None, T=0) == 0
    assert lib.gdn_last_error() == b""


def test_decode_rejects(lib):
    p = ctypes.c_void_p
    st = lib.gdn_decode_step(p(0x1000), p(0x2000), p(0x3000), p(0x4000), p(0x5000), None,
                             1, 1, 1, 128, 128, 1, p(0x6000), None)
    assert st == 1 and b"required" in lib.gdn_last_error()
    st = lib.gdn_decode_step(p(0x1000), p(0x2000), p(0x3000), p(0x4000), p(0x5000), p(0x10000),
                             1, 2, 3, 128, 128, 1, p(0x6000), None)
    assert st == 1


def test_plan(lib):
    plan = gdn.prefill_plan(1, 16, gdn.GDN_BF16, lib=lib)
    assert plan["workgroups"] * plan["dv_per_workgroup"] == 16 * 128
    assert 0 < plan["lds_bytes"] <= 160 * 1024
    assert plan["threads_per_workgroup"] in (256, 512)
    plan32 = gdn.prefill_plan(1, 1, gdn.GDN_F32, lib=lib)
    assert 0 < plan32["lds_bytes"] <= 160 * 1024
    assert plan32["threads_per_workgroup"] % 64 == 0
    # fp16 I/O runs the same pipelined kernel as bf16, with the same launch shape
    assert gdn.prefill_plan(1, 16, gdn.GDN_F16, lib=lib) == plan
    with pytest.raises(gdn.GDNError):
        gdn.prefill_plan(1, 16, 3, lib=lib)


@pytest.mark.parametrize("C", [32, 128])
def test_split_workspace_size_other_chunks(lib, C):
    # T_tot / C + N slots of C * 1024 + (C / 32) (C / 32 + 1) * 1024 + 512 bytes (the lower
    # triangle of P as 16x32 fragments)
    tile = C * 1024 + (C // 32) * (C // 32 + 1) * 1024 + 512
    assert gdn.prefill_split_workspace_size(1, 4096, 16, C, lib=lib) == (4096 // C + 1) * 16 * tile
    assert gdn.prefill_split_workspace_size(3, 100, 2, C, lib=lib) == (100 // C + 3) * 2 * tile
    with pytest.raises(gdn.GDNError):
        gdn.kda_workspace_size(1, 10, 1, chunk_size=C, lib=lib)


@pytest.mark.parametrize("size_fn", ["kda_workspace_size", "prefill_split_workspace_size"])
def test_workspace_size(lib, size_fn):
    # one 72,192-byte tile per value head and chunk slot, T_tot / 64 + N slots
    f = getattr(gdn, size_fn)
    assert f(1, 4096, 16, lib=lib) == (64 + 1) * 16 * 72192
    assert f(3, 100, 2, lib=lib) == (1 + 3) * 2 * 72192
    with pytest.raises(gdn.GDNError):
        f(1, 10, 1, chunk_size=48, lib=lib)


def _ws_prefill(lib, fn, **over):
    # fake, aligned, never-dereferenced addresses: validation fails before any use
    a = dict(q=0x100000, k=0x200000, v=0x300000, g=0x400000, beta=0x500000, s0=None, cu=None,
             N=1, T=10, Hk=2, Hv=4, Dk=128, Dv=128, C=64, io=1, ws=0x1000000, wsb=1 << 24,
             o=0x600000, fs=None)
    a.update(over)
    p = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return getattr(lib, fn)(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["s0"]),
                            p(a["cu"]), a["N"], a["T"], a["Hk"], a["Hv"], a["Dk"], a["Dv"], a["C"],
                            a["io"], p(a["ws"]), a["wsb"], p(a["o"]), p(a["fs"]), None)


def _kda_prefill(lib, **over):
    return _ws_prefill(lib, "gdn_kda_prefill", **over)


@pytest.mark.parametrize("over,status,msg", [
    (dict(io=0), 2, "bf16 or fp16"),
    (dict(C=128), 2, "chunk_size"),
    (dict(wsb=1000), 1, "smaller than"),
    (dict(ws=None), 1, "smaller than"),
    (dict(ws=0x1000080), 1, "256-byte aligned"),
    (dict(g=0x400008), 1, "g must be 16-byte aligned"),
    (dict(ws=0x300000), 1, "workspace overlaps v"),
    (dict(o=0x1000000), 1, "overlaps"),
    (dict(Hv=3), 1, "multiple"),
])
def test_kda_prefill_rejects(lib, over, status, msg):
    assert _kda_prefill(lib, **over) == status
    assert msg in lib.gdn_last_error().decode()


def test_kda_prefill_nothing_to_do_is_ok(lib):
    assert _kda_prefill(lib, q=None, k=None, v=None, g=None, beta=None, o=None, ws=None, wsb=0, T=0) == 0


@pytest.mark.parametrize("over,status,msg", [
    (dict(io=0), 2, "bf16 or fp16"),
    (dict(C=16), 2, "chunk_size"),
    (dict(C=256), 2, "chunk_size"),
    (dict(C=128, wsb=1 << 16), 1, "smaller than"),
    (dict(wsb=1000), 1, "smaller than"),
    (dict(ws=None), 1, "smaller than"),
    (dict(ws=0x1000080), 1, "256-byte aligned"),
    (dict(g=0x400002), 1, "g must be 4-byte aligned"),
    (dict(ws=0x500000), 1, "workspace overlaps beta"),
    (dict(fs=0x1000000), 1, "workspace overlaps an output"),
    (dict(N=2), 1, "cu_seqlens is required"),
])
def test_split_prefill_rejects(lib, over, status, msg):
    # the scalar gate's g is [T_tot, Hv] (4-byte aligned), as for gdn_prefill
    assert _ws_prefill(lib, "gdn_prefill_split", **over) == status
    assert msg in lib.gdn_last_error().decode()


def test_split_prefill_nothing_to_do_is_ok(lib):
    assert _ws_prefill(lib, "gdn_prefill_split", q=None, k=None, v=None, g=None, beta=None, o=None, ws=None,
                       wsb=0, T=0) == 0


def _noalloc(lib, **over):
    # fake, widely spaced, never-dereferenced addresses: validation fails before any use
    t = 1 << 40
    a = dict(q=t, k=2 * t, v=3 * t, g=4 * t, beta=5 * t, s0=None, cu=None, N=1, T=10, Hk=2, Hv=4,
             Dk=128, Dv=128, C=64, io=1, o=6 * t, fs=None)
    a.update(over)
    p = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lib.gdn_prefill_split_noalloc(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]),
                                         p(a["s0"]), p(a["cu"]), a["N"], a["T"], a["Hk"], a["Hv"], a["Dk"],
                                         a["Dv"], a["C"], a["io"], p(a["o"]), p(a["fs"]), None)


def _split_ws(lib, N, T, Hv, C):
    n = ctypes.c_size_t()
    assert lib.gdn_prefill_split_workspace_size(N, T, Hv, C, ctypes.byref(n)) == 0
    return n.value


@pytest.mark.parametrize("over,status,msg", [
    (dict(io=0), 2, "bf16 or fp16"),
    (dict(C=16), 2, "chunk_size"),
    (dict(g=4 * (1 << 40) + 2), 1, "g must be 4-byte aligned"),
    (dict(N=2), 1, "cu_seqlens is required"),
    # 64-token chunks: 1394 (slot, head) tiles fit in the 96 MiB scratch, 1395 do not
    (dict(T=(1395 - 1) * 64, Hv=1, Hk=1), 2, "static scratch"),
    (dict(T=1 << 20, Hv=16, Hk=16), 2, "static scratch"),
])
def test_split_noalloc_rejects(lib, over, status, msg):
    assert _noalloc(lib, **over) == status
    assert msg in lib.gdn_last_error().decode()


def test_split_noalloc_limit(lib):
    assert gdn.NOALLOC_SCRATCH_BYTES == 96 << 20
    # the largest single-head sequence that fits, and the H16 T4096 prefill
    assert _split_ws(lib, 1, (1394 - 1) * 64, 1, 64) <= gdn.NOALLOC_SCRATCH_BYTES
    assert _split_ws(lib, 1, 1394 * 64, 1, 64) > gdn.NOALLOC_SCRATCH_BYTES
    assert _split_ws(lib, 1, 4096, 16, 64) <= gdn.NOALLOC_SCRATCH_BYTES


def test_split_noalloc_nothing_to_do_is_ok(lib):
    assert _noalloc(lib, q=None, k=None, v=None, g=None, beta=None, o=None, T=0) == 0


def test_kda_decode_rejects(lib):
    p = ctypes.c_void_p
    # a per-channel gate must be 16-byte aligned
    st = lib.gdn_kda_decode_step(p(0x1000), p(0x2000), p(0x3000), p(0x4008), p(0x5000), p(0x10000),
                                 1, 1, 1, 128, 128, 1, p(0x60000), None)
    assert st == 1 and b"16-byte" in lib.gdn_last_error()
    # g of [B, Hv, 128] fp32 is 512 B: a state written at 0x4100 would overlap it
    st = lib.gdn_kda_decode_step(p(0x1000), p(0x2000), p(0x3000), p(0x4000), p(0x5000), p(0x4100),
                                 1, 1, 1, 128, 128, 1, p(0x60000), None)
    assert st == 1 and b"state overlaps g" in lib.gdn_last_error()


def _fused(lib, **over):
    a = dict(q=0x10000, k=0x20000, v=0x30000, g=0x40000, beta=0x50000, s0=None, cu=None,
             N=1, T=10, Hk=2, Hv=4, Dk=128, Dv=128, C=64, io=1, pro=7, o=0x60000, fs=None)
    a.update(over)
    p = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lib.gdn_prefill_fused(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["s0"]),
                                 p(a["cu"]), a["N"], a["T"], a["Hk"], a["Hv"], a["Dk"], a["Dv"], a["C"],
                                 a["io"], a["pro"], p(a["o"]), p(a["fs"]), None)


@pytest.mark.parametrize("over,status,msg", [
    (dict(pro=8), 1, "unknown bits"),
    (dict(io=0), 2, "bf16 or fp16"),
    (dict(C=32), 2, "chunk_size"),
    (dict(o=0x30000), 1, "overlaps"),
])
def test_prefill_fused_rejects(lib, over, status, msg):
    assert _fused(lib, **over) == status
    assert msg in lib.gdn_last_error().decode()


def test_decode_fused_rejects_unknown_flags(lib):
    p = ctypes.c_void_p
    st = lib.gdn_decode_step_fused(p(0x1000), p(0x2000), p(0x3000), p(0x4000), p(0x5000), p(0x10000),
                                   1, 1, 1, 128, 128, 1, 16, p(0x60000), None)
    assert st == 1 and b"unknown bits" in lib.gdn_last_error()


@pytest.mark.parametrize("C,K", [(64, 1), (64, 3), (32, 2), (128, 5)])
def test_seg_workspace_size(lib, C, K):
    # the split path's tiles, then o0 and e rows [T_tot, Hv, 128] (fp16), then per
    # (sequence, head, segment) two fp32 and one fp16 128 x 128 states
    for N, T, Hv in ((1, 4096, 16), (3, 100, 2), (2, 0, 1)):
        tiles = gdn.prefill_split_workspace_size(N, T, Hv, C, lib=lib)
        want = tiles + T * Hv * 128 * 2 * 2 + N * Hv * K * 128 * 128 * (2 * 4 + 2)
        assert gdn.prefill_seg_workspace_size(N, T, Hv, C, K, lib=lib) == want
    for bad in (0, 257, -1):
        with pytest.raises(gdn.GDNError):
            gdn.prefill_seg_workspace_size(1, 10, 1, 64, bad, lib=lib)
    with pytest.raises(gdn.GDNError):
        gdn.prefill_seg_workspace_size(1, 10, 1, 48, 1, lib=lib)


def _seg_prefill(lib, K=2, **over):
    a = dict(q=0x100000, k=0x200000, v=0x300000, g=0x400000, beta=0x500000, s0=None, cu=None,
             N=1, T=10, Hk=2, Hv=4, Dk=128, Dv=128, C=64, io=1, ws=0x1000000, wsb=1 << 24,
             o=0x600000, fs=None)
    a.update(over)
    p = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lib.gdn_prefill_seg(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["s0"]),
                               p(a["cu"]), a["N"], a["T"], a["Hk"], a["Hv"], a["Dk"], a["Dv"], a["C"], K,
                               a["io"], p(a["ws"]), a["wsb"], p(a["o"]), p(a["fs"]), None)


@pytest.mark.parametrize("K,over,status,msg", [
    (0, {}, 1, "segments=0"),
    (300, {}, 1, "segments=300"),
    (2, dict(io=0), 2, "bf16 or fp16"),
    (2, dict(C=16), 2, "chunk_size"),
    (2, dict(wsb=1 << 18), 1, "smaller than"),
    (2, dict(ws=None), 1, "smaller than"),
    (2, dict(ws=0x1000080), 1, "256-byte aligned"),
    (2, dict(ws=0x500000), 1, "workspace overlaps beta"),
    (2, dict(fs=0x1000000), 1, "workspace overlaps an output"),
    (2, dict(N=2), 1, "cu_seqlens is required"),
])
def test_seg_prefill_rejects(lib, K, over, status, msg):
    assert _seg_prefill(lib, K, **over) == status
    assert msg in lib.gdn_last_error().decode()


def test_seg_prefill_nothing_to_do_is_ok(lib):
    assert _seg_prefill(lib, 3, q=None, k=None, v=None, g=None, beta=None, o=None, ws=None, wsb=0, T=0) == 0


def test_seg_choose_needs_a_device(lib):
    # the count depends on the device's compute units; without a GPU it is a device error
    K = ctypes.c_int32(-1)
    assert lib.gdn_prefill_seg_choose(1, 4096, 4, 64, None) == 1
    assert lib.gdn_prefill_seg_choose(1, 4096, 4, 48, ctypes.byref(K)) == 2
    st = lib.gdn_prefill_seg_choose(1, 4096, 4, 64, ctypes.byref(K))
    if torch.cuda.is_available():
        assert st == 0 and K.value >= 1
    else:
        assert st == 3 and b"compute-unit" in lib.gdn_last_error()


def _split_fused(lib, pro, **over):
    a = dict(q=0x100000, k=0x200000, v=0x300000, g=0x400000, beta=0x500000, s0=None, cu=None,
             N=1, T=10, Hk=2, Hv=4, Dk=128, Dv=128, C=64, io=1, ws=0x1000000, wsb=1 << 24,
             o=0x600000, fs=None)
    a.update(over)
    p = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lib.gdn_prefill_split_fused(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["s0"]),
                                       p(a["cu"]), a["N"], a["T"], a["Hk"], a["Hv"], a["Dk"], a["Dv"], a["C"],
                                       a["io"], pro, p(a["ws"]), a["wsb"], p(a["o"]), p(a["fs"]), None)


@pytest.mark.parametrize("pro,over,status,msg", [
    (8, {}, 1, "unknown bits"),
    (7, dict(io=0), 2, "bf16 or fp16"),
    (7, dict(C=16), 2, "chunk_size"),
    (7, dict(wsb=1000), 1, "smaller than"),
    (7, dict(o=0x300000), 1, "overlaps"),
])
def test_split_fused_rejects(lib, pro, over, status, msg):
    assert _split_fused(lib, pro, **over) == status
    assert msg in lib.gdn_last_error().decode()


def test_split_fused_nothing_to_do_is_ok(lib):
    assert _split_fused(lib, 7, q=None, k=None, v=None, g=None, beta=None, o=None, ws=None, wsb=0, T=0) == 0


@pytest.mark.parametrize("over,status,msg", [
    (dict(C=32), 2, "chunk_size"),
    (dict(g=0x400008), 1, "g must be 16-byte aligned"),
    (dict(io=0), 2, "bf16 or fp16"),
    (dict(wsb=1 << 18), 1, "smaller than"),
])
def test_kda_seg_rejects(lib, over, status, msg):
    a = dict(q=0x100000, k=0x200000, v=0x300000, g=0x400000, beta=0x500000, s0=None, cu=None,
             N=1, T=10, Hk=2, Hv=4, Dk=128, Dv=128, C=64, io=1, ws=0x1000000, wsb=1 << 24,
             o=0x600000, fs=None)
    a.update(over)
    p = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    st = lib.gdn_kda_prefill_seg(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["s0"]),
                                 p(a["cu"]), a["N"], a["T"], a["Hk"], a["Hv"], a["Dk"], a["Dv"], a["C"], 2,
                                 a["io"], p(a["ws"]), a["wsb"], p(a["o"]), p(a["fs"]), None)
    assert st == status
    assert msg in lib.gdn_last_error().decode()


def _auto_plan(lib, N=1, T=4096, Hv=16, io=1, pro=0, want_bytes=True):
    path, seg, n = ctypes.c_int32(-1), ctypes.c_int32(-1), ctypes.c_size_t(7)
    st = lib.gdn_prefill_auto_plan(N, T, Hv, io, pro, ctypes.byref(path), ctypes.byref(seg),
                                   ctypes.byref(n) if want_bytes else None)
    return st, path.value, seg.value, n.value


def test_auto_plan_fp32_is_the_one_launch_path(lib):
    # fp32 I/O has one path, chosen without asking the device
    assert _auto_plan(lib, io=0) == (0, gdn.PATH_ONE_LAUNCH, 1, 0)


@pytest.mark.parametrize("over,status,msg", [
    (dict(io=5), 1, "io_dtype"),
    (dict(N=0), 1, "out of range"),
    (dict(T=-1), 1, "out of range"),
    (dict(pro=8), 1, "unknown bits"),
    (dict(want_bytes=False), 1, "workspace_bytes must be non-null"),
])
def test_auto_plan_rejects(lib, over, status, msg):
    assert _auto_plan(lib, **over)[0] == status
    assert msg in lib.gdn_last_error().decode()


def test_auto_plan_needs_a_device_for_16_bit_io(lib):
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _auto_plan(lib)[0] == 3
    assert "compute-unit count" in lib.gdn_last_error().decode()


def test_auto_rejects_before_planning_nothing(lib):
    p = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    st = lib.gdn_prefill_auto(p(0x100000), p(0x200000), p(0x300000), p(0x400000), p(0x500000), None, None,
                              1, 10, 2, 4, 128, 128, 0, 9, None, 0, p(0x600000), None, None)
    assert st == 1 and "unknown bits" in lib.gdn_last_error().decode()


def test_gdn_check_reads_cu_seqlens_before_any_launch(lib, monkeypatch):
    # without a GPU the read-back itself fails: the check runs first, after the host
    # checks and before any launch, and says so
    if torch.cuda.is_available():
        pytest.skip("a GPU is present (the GPU tests cover malformed cu_seqlens)")
    p = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    args = lambda: (p(0x100000), p(0x200000), p(0x300000), p(0x400000), p(0x500000), None, p(0x700000),  # noqa: E731
                    2, 10, 2, 4, 128, 128, 64, 1, p(0x600000), None, None)
    monkeypatch.setenv("GDN_CHECK", "1")
    assert lib.gdn_prefill(*args()) == 3
    assert "GDN_CHECK: reading cu_seqlens back failed" in lib.gdn_last_error().decode()
    monkeypatch.setenv("GDN_CHECK", "0")
    lib.gdn_prefill(*args())
    assert "GDN_CHECK" not in lib.gdn_last_error().decode()
