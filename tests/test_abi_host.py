"""The C-ABI library on the host: symbols, blob packing, and argument checks
that run before any HIP call (no GPU needed)."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

from block_scaled_fp4_gemv_amd import binding as B
from block_scaled_fp4_gemv_amd import synth as sy

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 15
    L = ctypes.CDLL(B.LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(L, n)]
    assert not missing, missing
    assert set(B.SIGNATURES) == names


def test_status_strings():
    assert B.lib().moe_status_str(0) == b"ok"
    assert B.lib().moe_status_str(B.MOE_E_CAPACITY) == b"cache capacity exceeded"
    assert B.lib().moe_abi_version() == (1 << 16) | 2   # 1.2: prepared routers (MOE_ROUTE_PREPARED)


@pytest.mark.parametrize("fmt,H,F,exp", [
    (1, 2048, 512, 3 * 524288 + 3 * 65536 + 256),
    (2, 256, 512, 3 * 65536 + 2 * 4096 + 4096 + 256),
    (3, 6144, 2048, 3 * 12582912 + 3 * 393216 + 256),
])
def test_expert_bytes(fmt, H, F, exp):
    assert B.moe_expert_bytes(fmt, H, F) == exp


@pytest.mark.parametrize("bad", [(0, 2048, 512), (4, 2048, 512), (1, 2000, 512), (1, 2048, 96)])
def test_expert_bytes_invalid(bad):
    assert B.moe_expert_bytes(*bad) == 0


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_pack_unpack_round_trip(fmt):
    H, F = 256, 512
    b = sy.experts(fmt, 0, 5, 0, 0, 1, H, F, 0.02)
    canon = sy.expert_view(b, 0)
    blob = B.moe_pack_expert(fmt, H, F, canon)
    back = B.moe_unpack_expert(fmt, H, F, blob)
    for key in ("codes_g", "codes_u", "codes_d", "scales_g", "scales_u", "scales_d"):
        assert np.array_equal(back[key], canon[key]), key
    if fmt == 1:
        assert (back["tau_g"], back["tau_u"], back["tau_d"]) == (canon["tau_g"], canon["tau_u"], canon["tau_d"])
    else:
        assert back["tau_g"] == 1.0
    # every section holds the fragment order the header documents, 256-aligned
    assert np.array_equal(blob, _documented_blob(fmt, H, F, canon))


def _frag_order(fmt, a, is_scale):
    """Canonical [N][...] array -> bytes in the documented fragment order: row
    groups of 16, steps of 128 k, lane l = 16*q + r owning k 32q..32q+31 of the step."""
    N = a.shape[0]
    if not is_scale:
        if fmt == 3:   # bytes k = 128s + 32q + 16p + j -> [g][s][p][q][r][j]
            v = a.reshape(N // 16, 16, -1, 4, 2, 16).transpose(0, 2, 4, 3, 1, 5)
        else:          # bytes 64s + 16q + j -> [g][s][q][r][j]
            v = a.reshape(N // 16, 16, -1, 4, 16).transpose(0, 2, 3, 1, 4)
    elif fmt == 1:     # scale 8s + 2q + b -> [g][s][q][r][b]
        v = a.reshape(N // 16, 16, -1, 4, 2).transpose(0, 2, 3, 1, 4)
    elif fmt == 2:     # scale 4s + q -> [g][s][q][r]
        v = a.reshape(N // 16, 16, -1, 4).transpose(0, 2, 3, 1)
    else:              # fp32 scale s -> [g][s][r]
        v = a.reshape(N // 16, 16, -1).transpose(0, 2, 1)
    return np.ascontiguousarray(v).view(np.uint8).ravel()


def _documented_blob(fmt, H, F, canon):
    out = np.zeros(B.moe_expert_bytes(fmt, H, F), np.uint8)
    pos = 0
    for key in ("codes_g", "codes_u", "codes_d", "scales_g", "scales_u", "scales_d"):
        b = _frag_order(fmt, np.asarray(canon[key]), key.startswith("scales"))
        out[pos:pos + b.size] = b
        pos = (pos + b.size + 255) // 256 * 256
    tau = [canon["tau_g"], canon["tau_u"], canon["tau_d"]] if fmt == 1 else [1.0, 1.0, 1.0]
    out[pos:pos + 12] = np.asarray(tau, np.float32).view(np.uint8)
    return out


def test_pack_rejects_null():
    ptrs = (ctypes.c_void_p * 9)()
    blob = np.zeros(B.moe_expert_bytes(1, 256, 512), np.uint8)
    assert B.lib().moe_pack_expert(1, 256, 512, ptrs, blob.ctypes.data) == B.MOE_E_ARG
    assert B.lib().moe_pack_expert(9, 256, 512, ptrs, blob.ctypes.data) == B.MOE_E_FORMAT


def test_route_argument_errors_before_any_hip_call():
    L = B.lib()
    ws = np.zeros(1 << 20, np.uint8)
    fake = 0x1000  # never dereferenced: validation fails first
    args = lambda T, H, E, k, flags=0, ws_bytes=ws.nbytes, perm=None, off=None: (  # noqa: E731
        fake, fake, T, H, E, k, flags, fake, fake, perm, off, ws.ctypes.data, ws_bytes, None)
    assert L.moe_route(*args(1, 2048, 256, 0)) == B.MOE_E_ARG          # k < 1
    assert L.moe_route(*args(1, 2048, 4, 5)) == B.MOE_E_ARG            # k > E
    assert L.moe_route(*args(1, 2048, 2048, 8)) == B.MOE_E_ARG         # E > 1024
    assert L.moe_route(*args(1, 1000, 256, 8)) == B.MOE_E_ARG          # H unsupported
    assert L.moe_route(*args(-1, 2048, 256, 8)) == B.MOE_E_ARG
    assert L.moe_route(*args(1, 2048, 256, 8, flags=4)) == B.MOE_E_ARG
    assert L.moe_route(*args(1, 2048, 256, 8, perm=fake)) == B.MOE_E_ARG   # perm without off
    assert L.moe_route(*args(64, 2048, 256, 8, ws_bytes=16)) == B.MOE_E_WORKSPACE
    assert b"workspace" in L.moe_last_error()


def test_ffn_argument_errors_before_any_hip_call():
    L = B.lib()
    fake = 0x100000
    eb = B.blob_stride(1, 2048, 512)
    raw = np.zeros((1 << 22) + 256, np.uint8)
    ws = raw[(-raw.ctypes.data) % 256:][: 1 << 22]
    def call(fmt=1, stride=eb, H=2048, F=512, E=256, T=1, k=8, y=fake, out=None, w=None,
             subset=None, n_sub=0, flags=0, ws_bytes=ws.nbytes, perm=None, off=None):
        return L.moe_expert_ffn(fmt, fake, stride, H, F, E, fake, T, k, fake, None, perm, off, subset,
                                n_sub, w, y, out, flags, ws.ctypes.data, ws_bytes, None)
    assert call(fmt=7) == B.MOE_E_FORMAT
    assert call(H=3000) == B.MOE_E_ARG
    assert call(stride=eb - 256) == B.MOE_E_ARG
    assert call(stride=eb + 1) == B.MOE_E_ARG
    assert call(y=None, out=None) == B.MOE_E_ARG
    assert call(out=fake, w=None) == B.MOE_E_ARG
    assert call(out=fake, w=fake, subset=fake, n_sub=1) == B.MOE_E_ARG
    assert call(flags=B.MOE_FFN_GROUPED) == B.MOE_E_ARG              # no permutation
    assert call(k=300) == B.MOE_E_ARG
    assert call(ws_bytes=8) == B.MOE_E_WORKSPACE
    assert call(k=32, E=64, out=fake, w=fake, flags=B.MOE_FFN_GEMV) == B.MOE_E_ARG   # k <= 16


def test_combine_and_lru_argument_errors():
    L = B.lib()
    assert L.moe_combine(0x1000, 0x1000, 1, 100, 8, 0x1000, None) == B.MOE_E_ARG
    assert L.moe_combine(0x1004, 0x1000, 1, 2048, 8, 0x1000, None) == B.MOE_E_ARG   # misaligned y
    st = B.moe_lru(256, 64, None, None, None, None)
    assert L.moe_lru_reset(ctypes.byref(st), None) == B.MOE_E_ARG
    st2 = B.moe_lru(256, 4096, 0x1000, 0x1000, 0x1000, 0x1000)
    assert L.moe_cache_lookup(ctypes.byref(st2), 0x1000, 1, 8, 0x1000, 0x1000, 0x1000, None) == B.MOE_E_ARG
    assert B.moe_miss_record_words(1, 8, 64) == 5 + 16
    assert B.moe_miss_record_words(16, 8, 64) == 5 + 128


def test_cache_fill_refuses_capacity_record():
    rec = np.array([B.MOE_E_CAPACITY, 3, 0, 0, 2, 0, 0, 0, 0], np.int32)
    L = B.lib()
    assert L.moe_cache_fill(rec.ctypes.data, 0x1000, 0x1000, 256, 256, None, None, None) == B.MOE_E_CAPACITY
    rec_bad = np.array([0, 5, 0, 0, 2, 0, 0, 0, 0], np.int32)   # n_miss > n_max
    assert L.moe_cache_fill(rec_bad.ctypes.data, 0x1000, 0x1000, 256, 256, None, None, None) == B.MOE_E_ARG


def test_cached_layer_argument_errors_before_any_hip_call():
    L = B.lib()
    fmt, H, F, E, k, T = 1, 2048, 512, 256, 8, 1
    need = B.moe_cached_layer_workspace(fmt, T, H, F, k, E)
    y = (T * k * H * 4 + 255) // 256 * 256
    assert need == y + (B.moe_route_workspace(T, H, E, k) + 255) // 256 * 256 + \
        B.lib().moe_ffn_workspace(fmt, T, H, F, k, E)
    assert B.moe_cached_layer_workspace(fmt, T, 2000, F, k, E) == 0
    fake = 0x1000  # never dereferenced: validation fails first
    h = ctypes.c_int32(0)

    def call(layer, ws_bytes):
        return L.moe_cached_layer_forward(fmt, B.blob_stride(fmt, H, F), H, F, E, k, 0, layer, fake, T, fake,
                                          fake, fake, fake, fake, 0x100000, ws_bytes, None, None,
                                          ctypes.byref(h), ctypes.byref(h))
    assert call(None, need) == B.MOE_E_ARG
    layer = B.moe_cached_layer(fake, fake, fake, B.moe_lru(E, 64, fake, fake, fake, fake), fake, fake, None, None)
    assert call(ctypes.byref(layer), need - 1) == B.MOE_E_WORKSPACE


def test_prefill_streamed_argument_errors_before_any_hip_call():
    L = B.lib()
    fmt, H, F, E, k, T, n = 2, 2048, 512, 256, 8, 64, 3
    need = B.moe_prefill_streamed_workspace(fmt, T, H, F, k, E)
    assert need == B.lib().moe_layer_workspace(fmt, T, H, F, k, E) > 0
    fake = 0x1000  # never dereferenced: validation fails first
    vp = ctypes.c_void_p
    arr = lambda m, v=fake: (vp * m)(*([v] * m))  # noqa: E731
    pools = (vp * 2)(fake, fake + 0x100000)
    stride = B.blob_stride(fmt, H, F)

    def call(events, ws_bytes, s=0x11, cs=0x22, pools=pools, layers=n):
        return L.moe_prefill_streamed(fmt, stride, H, F, E, k, 0, layers, arr(n), arr(n), fake, T, arr(n), fake,
                                      fake, pools, 0x100000, ws_bytes, s, cs, events)
    assert call(arr(4), need - 1) == B.MOE_E_WORKSPACE
    assert call(arr(4, None), need) == B.MOE_E_ARG            # NULL events
    assert call(arr(4), need, cs=0x11) == B.MOE_E_ARG          # copy stream == stream
    assert call(arr(4), need, pools=(vp * 2)(fake, fake)) == B.MOE_E_ARG
    assert call(arr(4), need, layers=-1) == B.MOE_E_ARG
    assert call(arr(4), need, layers=0) == B.MOE_OK            # nothing to do


def test_layer_forward_prefetch_argument_errors_before_any_hip_call():
    """The read-ahead hint is both set or both absent, and 16-byte aligned; the
    checks run before any HIP call (fake addresses are never dereferenced)."""
    L = B.lib()
    fmt, H, F, E, k, T = 1, 2048, 512, 256, 8, 1
    need = L.moe_layer_workspace(fmt, T, H, F, k, E)
    stride = B.blob_stride(fmt, H, F)
    fake = 0x100000

    def call(warm, warm_bytes, ws_bytes=need):
        return L.moe_layer_forward_prefetch(fmt, fake, stride, H, F, E, k, 0, fake, T, fake, fake, fake, fake,
                                            fake, ws_bytes, warm, warm_bytes, None)
    assert call(None, 64) == B.MOE_E_ARG           # bytes without a buffer
    assert call(fake, 0) == B.MOE_E_ARG            # buffer without bytes
    assert call(fake + 8, 64) == B.MOE_E_ARG       # misaligned
    assert call(fake, 64, need - 1) == B.MOE_E_WORKSPACE
    assert L.moe_layer_forward_prefetch(fmt, fake, stride, H, F, E, k, 0, fake, 0, fake, fake, fake, fake,
                                        fake, need, fake, 64, None) == B.MOE_OK   # T = 0: nothing to do


def test_lru_resize_argument_errors_before_any_hip_call():
    """moe_lru_resize checks states, pools, sizes and the workspace on the host
    (fake addresses are never dereferenced: every case fails before a launch)."""
    L = B.lib()
    fake, eb, stride = 0x10000000, 1769728, 1769728
    st = lambda E, S, p=fake: B.moe_lru(E, S, p, p, p, p)  # noqa: E731
    need = L.moe_lru_resize_workspace(32)
    assert need >= (1 + 2 * 32) * 4 and need % 256 == 0
    assert L.moe_lru_resize_workspace(0) == 0 and L.moe_lru_resize_workspace(1025) == 0

    def call(a, pa, b, pb, e=eb, s=stride, ws=fake, wsb=need):
        return L.moe_lru_resize(ctypes.byref(a), pa, ctypes.byref(b), pb, e, s, ws, wsb, None)
    other = fake + 64 * stride                                     # a second, disjoint pool
    assert call(st(256, 64, None), fake, st(256, 32), other) == B.MOE_E_ARG    # NULL state arrays
    assert call(st(256, 64), fake, st(256, 0), other) == B.MOE_E_ARG           # S < 1
    assert call(st(256, 64), fake, st(256, 1025), other) == B.MOE_E_ARG        # S > 1024
    assert call(st(256, 64), fake, st(128, 32), other) == B.MOE_E_ARG          # E changed
    assert call(st(256, 64), None, st(256, 32), other) == B.MOE_E_ARG          # NULL pool
    assert call(st(256, 64), fake, st(256, 32), other, e=eb + 16) == B.MOE_E_ARG   # not a multiple of 256
    assert call(st(256, 64), fake, st(256, 32), other, s=eb - 256) == B.MOE_E_ARG  # stride < expert_bytes
    assert call(st(256, 64), fake + 8, st(256, 32), other) == B.MOE_E_ARG      # misaligned pool
    assert call(st(256, 64), fake, st(256, 32), fake + stride) == B.MOE_E_ARG  # partly overlapping pools
    assert call(st(256, 64), fake, st(256, 32), other, wsb=need - 1) == B.MOE_E_WORKSPACE
    assert call(st(256, 64), fake, st(256, 32), other, ws=None) == B.MOE_E_WORKSPACE


def test_layer_forward_static_checks_before_any_hip_call():
    """The allocation-free layer call refuses bad arguments and a workspace larger
    than its static array on the host, without touching a GPU."""
    L = B.lib()
    fmt, H, E, F, k = 1, 2048, 256, 512, 8
    stride = B.blob_stride(fmt, H, F)
    fake = 1 << 20                      # an aligned address that is never dereferenced
    # 2048 tokens need ~155 MiB of workspace: more than the 32 MiB array
    assert L.moe_layer_forward_static(fmt, fake, stride, H, F, E, k, 0, fake, 2048, fake, fake, fake, fake,
                                      None) == B.MOE_E_WORKSPACE
    assert L.moe_layer_forward_static(fmt, None, stride, H, F, E, k, 0, fake, 1, fake, fake, fake, fake,
                                      None) == B.MOE_E_ARG
    assert L.moe_layer_forward_static(fmt, fake, stride, H, F, E, k, 0, None, 1, fake, fake, fake, fake,
                                      None) == B.MOE_E_ARG
    assert L.moe_layer_forward_static(fmt, fake, stride + 16, H, F, E, k, 0, fake, 1, fake, fake, fake, fake,
                                      None) == B.MOE_E_ARG
    assert L.moe_layer_forward_static(9, fake, stride, H, F, E, k, 0, fake, 1, fake, fake, fake, fake,
                                      None) == B.MOE_E_FORMAT
    assert L.moe_layer_forward_static(fmt, fake, stride, H, F, E, k, 0, fake, 0, fake, fake, fake, fake,
                                      None) == B.MOE_OK


def test_router_prepare_sizes_and_argument_errors():
    """moe_router_prepared_bytes = 256-aligned fp32 router + 256-aligned three
    bf16 planes; moe_router_prepare and the route calls refuse bad arguments
    before any HIP call."""
    L = B.lib()
    for E, H in ((8, 256), (256, 2048), (256, 6144), (1024, 8192)):
        a = (E * H * 4 + 255) // 256 * 256
        assert B.lib().moe_router_prepared_bytes(E, H) == a + (3 * E * H * 2 + 255) // 256 * 256
    assert L.moe_router_prepared_bytes(0, 2048) == 0
    assert L.moe_router_prepared_bytes(1025, 2048) == 0
    assert L.moe_router_prepared_bytes(256, 300) == 0
    assert L.moe_router_prepare(0x1000, 0, 2048, 0x1000, None) == B.MOE_E_ARG     # E
    assert L.moe_router_prepare(None, 256, 2048, 0x1000, None) == B.MOE_E_ARG     # NULL router
    assert L.moe_router_prepare(0x1000, 256, 2048, None, None) == B.MOE_E_ARG     # NULL buffer
    assert L.moe_router_prepare(0x1004, 256, 2048, 0x1000, None) == B.MOE_E_ARG   # router not 16-aligned
    assert L.moe_router_prepare(0x1000, 256, 2048, 0x1010, None) == B.MOE_E_ARG   # buffer not 256-aligned
    # an unknown route flag next to MOE_ROUTE_PREPARED is refused by the route call
    ws = np.zeros(B.moe_route_workspace(8, 2048, 256, 8) + 256, np.uint8)
    wsp = (ws.ctypes.data + 255) // 256 * 256
    assert L.moe_route(0x1000, 0x1000, 8, 2048, 256, 8, B.MOE_ROUTE_PREPARED | 0x400, 0x1000, 0x1000,
                       None, None, wsp, ws.size - 256, None) == B.MOE_E_ARG
