"""Seeded synthetic inputs (bindings to ``libsynth.so``, built from synth.c).

Inputs only: normal draws, bf16 activations, AR(1) decode states and the
quantization of fp32 expert weights into canonical NVFP4 / MXFP4 / FP8 bytes.
Nothing here computes any part of the layer; both the GPU path and the CPU
checker consume what this module writes.
"""

import ctypes
import os

import numpy as np

from .workloads import WORKLOADS, Workload  # noqa: F401

NVFP4, MXFP4, FP8 = 1, 2, 3
KIND_X, KIND_ROUTER, KIND_W, KIND_EPS, KIND_H0 = 1, 2, 3, 4, 5
DEFAULT_SEED = 0

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        u64, u32, i32, sz, dbl = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                  ctypes.c_size_t, ctypes.c_double)
        vp = ctypes.c_void_p
        L.synth_stream.restype = u64
        L.synth_stream.argtypes = [u64, u32, u32, u32, u32, u32, u32]
        L.synth_normal.argtypes = [u64, u64, sz, dbl, dbl, vp]
        L.synth_normal_bf16.argtypes = [u64, u64, sz, dbl, dbl, vp]
        L.synth_f32_to_bf16.argtypes = [vp, sz, vp]
        L.synth_ar1_bf16.argtypes = [vp, vp, sz, dbl, dbl, vp]
        L.synth_quantize.restype = i32
        L.synth_quantize.argtypes = [i32, vp, i32, i32, vp, vp, vp]
        L.synth_experts.restype = i32
        L.synth_experts.argtypes = [i32, u64, u32, u32, u32, i32, i32, i32, dbl,
                                    vp, vp, vp, vp, vp, vp, vp]
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        L.synth_e2m1_encode.restype = ctypes.c_uint8
        L.synth_e2m1_encode.argtypes = [dbl]
        L.synth_e4m3_encode.restype = ctypes.c_uint8
        L.synth_e4m3_encode.argtypes = [dbl]
        L.synth_set_threads.argtypes = [i32]
        L.synth_get_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int):
    lib().synth_set_threads(int(n))


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def e2m1_encode(v: float) -> int:
    return int(lib().synth_e2m1_encode(float(v)))


def e4m3_encode(v: float) -> int:
    return int(lib().synth_e4m3_encode(float(v)))


def stream(seed, cfg, kind, layer=0, expert=0, matrix=0, attempt=0) -> int:
    return int(lib().synth_stream(seed, cfg, kind, layer, expert, matrix, attempt))


def normal(st: int, n: int, mean=0.0, std=1.0, first=0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal(st, first, n, mean, std, _p(out))
    return out


def normal_bf16(st: int, n: int, mean=0.0, std=1.0, first=0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().synth_normal_bf16(st, first, n, mean, std, _p(out))
    return out


def f32_to_bf16(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().synth_f32_to_bf16(_p(a), a.size, _p(out))
    return out


def quantize(fmt: int, w) -> dict:
    """fp32 [N, K] -> canonical dict(codes, scales, tau)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if fmt == FP8:
        codes = np.empty((N, K), dtype=np.uint8)
        scales = np.empty((N, K // 128), dtype=np.float32)
    else:
        codes = np.empty((N, K // 2), dtype=np.uint8)
        scales = np.empty((N, K // (16 if fmt == NVFP4 else 32)), dtype=np.uint8)
    tau = np.ones(1, dtype=np.float32)
    if lib().synth_quantize(fmt, _p(w), N, K, _p(codes), _p(scales), _p(tau)) != 0:
        raise ValueError("bad quantize shape")
    return dict(codes=codes, scales=scales, tau=np.float32(tau[0]))


def _code_shape(fmt, N, K):
    return (N, K) if fmt == FP8 else (N, K // 2)


def _scale_shape_dtype(fmt, N, K):
    if fmt == NVFP4:
        return (N, K // 16), np.uint8
    if fmt == MXFP4:
        return (N, K // 32), np.uint8
    return (N, K // 128), np.float32


def experts(fmt, seed, cfg, layer, e0, n, H, F, std) -> dict:
    """Canonical bytes of experts e0..e0+n-1 of one layer (leading axis = expert)."""
    cg = np.empty((n,) + _code_shape(fmt, F, H), dtype=np.uint8)
    cu = np.empty_like(cg)
    cd = np.empty((n,) + _code_shape(fmt, H, F), dtype=np.uint8)
    sshape, sdt = _scale_shape_dtype(fmt, F, H)
    sg = np.empty((n,) + sshape, dtype=sdt)
    su = np.empty_like(sg)
    dshape, _ = _scale_shape_dtype(fmt, H, F)
    sd = np.empty((n,) + dshape, dtype=sdt)
    tau = np.empty((n, 3), dtype=np.float32)
    r = lib().synth_experts(fmt, seed, cfg, layer, e0, n, H, F, float(std), _p(cg), _p(cu), _p(cd),
                            _p(sg), _p(su), _p(sd), _p(tau))
    if r != 0:
        raise ValueError("bad expert shape")
    return dict(codes_g=cg, codes_u=cu, codes_d=cd, scales_g=sg, scales_u=su, scales_d=sd, tau=tau)


def expert_view(batch: dict, i: int) -> dict:
    """One expert's canonical dict from an ``experts`` batch."""
    d = {k: batch[k][i] for k in ("codes_g", "codes_u", "codes_d", "scales_g", "scales_u", "scales_d")}
    d["tau_g"], d["tau_u"], d["tau_d"] = (np.float32(batch["tau"][i, j]) for j in range(3))
    return d


class ExpertList:
    """Indexable view over an ``experts`` batch: ``lst[e]`` -> canonical dict."""

    def __init__(self, batch):
        self.batch = batch

    def __getitem__(self, e):
        return expert_view(self.batch, int(e))

    def __len__(self):
        return self.batch["codes_g"].shape[0]


def router(seed, cfg, layer, E, H, std=0.05) -> np.ndarray:
    st = stream(seed, cfg, KIND_ROUTER, layer)
    return normal(st, E * H, 0.0, std).reshape(E, H)


def router_skewed(seed, cfg, layer, E, H, sigma, std=0.05) -> np.ndarray:
    """router() with row e scaled by exp(sigma * g_e), g_e ~ N(0, 1) from its own
    stream: larger sigma concentrates a layer's routing on fewer experts (a
    smaller working set), sigma = 0 is router() itself."""
    g = normal(stream(seed, cfg, KIND_ROUTER, layer, 0, 1), E)
    r = router(seed, cfg, layer, E, H, std)
    return (r * np.exp(sigma * g)[:, None]).astype(np.float32)


def token_row(seed, cfg, t, H, attempt=0, std=1.0) -> np.ndarray:
    """bf16 row t of an i.i.d. N(0, std^2) token batch (redrawn with attempt+1)."""
    return normal_bf16(stream(seed, cfg, KIND_X, 0, t, 0, attempt), H, 0.0, std)


def token_rows(seed, cfg, T, H, attempts=None, std=1.0) -> np.ndarray:
    out = np.empty((T, H), dtype=np.uint16)
    for t in range(T):
        out[t] = token_row(seed, cfg, t, H, 0 if attempts is None else int(attempts[t]), std)
    return out


def ar1_h0(seed, cfg, H) -> np.ndarray:
    return normal_bf16(stream(seed, cfg, KIND_H0), H)


def ar1_next(h_prev, seed, cfg, t, H, attempt=0, rho=0.9, c=0.44) -> np.ndarray:
    """h_t = bf16(rho * h_{t-1} + c * eps_t), eps_t ~ N(0,1) from stream (EPS, t, attempt)."""
    eps = normal(stream(seed, cfg, KIND_EPS, 0, t, 0, attempt), H)
    h_prev = np.ascontiguousarray(h_prev, dtype=np.uint16)
    out = np.empty(H, dtype=np.uint16)
    lib().synth_ar1_bf16(_p(h_prev), _p(eps), H, rho, c, _p(out))
    return out


def ar1_sequence(seed, cfg, n_steps, H, attempts=None) -> np.ndarray:
    """Decode states h_0..h_{n-1} (bf16 [n, H]); attempts[t] redraws eps_t."""
    out = np.empty((n_steps, H), dtype=np.uint16)
    h = ar1_h0(seed, cfg, H)
    if attempts is not None and attempts[0]:
        h = normal_bf16(stream(seed, cfg, KIND_H0, 0, 0, 0, int(attempts[0])), H)
    out[0] = h
    for t in range(1, n_steps):
        h = ar1_next(h, seed, cfg, t, H, 0 if attempts is None else int(attempts[t]))
        out[t] = h
    return out
