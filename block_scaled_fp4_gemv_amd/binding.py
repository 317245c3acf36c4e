"""ctypes binding of ``libmoe_fp4.so`` (the C ABI in include/moe_fp4.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Device buffers are torch CUDA tensors (PyTorch supplies device
memory and streams); host blobs are numpy arrays.  Functions keep the C
names.  Output tensors that the caller does not pass are allocated here with
torch (the library itself never allocates).  A missing library raises.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp4.so")

MOE_OK, MOE_E_ARG, MOE_E_FORMAT, MOE_E_CAPACITY, MOE_E_WORKSPACE, MOE_E_HIP = 0, -1, -2, -3, -4, -5
MOE_FMT_NVFP4, MOE_FMT_MXFP4, MOE_FMT_FP8_E4M3 = 1, 2, 3
MOE_ROUTE_RENORM = 1
MOE_ROUTE_PREPARED = 0x200      # router is a prepared router (moe_router_prepare)
MOE_FFN_AUTO, MOE_FFN_GEMV, MOE_FFN_GROUPED = 0, 1, 2
MOE_FFN_MX_NATIVE = 4           # MXFP4 grouped path on the scaled MFMA (FP8 activation terms)
MOE_LAYER_MX_NATIVE = 0x100     # the same for moe_layer_forward (in its route flags)

_vp, _i32, _u32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t


class moe_lru(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("S", ctypes.c_int32), ("slot_expert", _vp),
                ("expert_slot", _vp), ("slot_stamp", _vp), ("clock", _vp), ("key_base", ctypes.c_int32)]


class moe_cached_layer(ctypes.Structure):
    _fields_ = [("router", _vp), ("host_pool", _vp), ("slot_pool", _vp), ("lru", moe_lru),
                ("miss_rec", _vp), ("lookup_done", _vp), ("slots_free", _vp), ("fill_done", _vp)]


SIGNATURES = {
    "moe_status_str": (ctypes.c_char_p, [_i32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (_i32, []),
    "moe_expert_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_pack_expert": (_i32, [_i32, _i32, _i32, ctypes.POINTER(_vp), _vp]),
    "moe_unpack_expert": (_i32, [_i32, _i32, _i32, _vp, ctypes.POINTER(_vp)]),
    "moe_route_workspace": (_sz, [_i32, _i32, _i32, _i32]),
    "moe_router_prepared_bytes": (_sz, [_i32, _i32]),
    "moe_router_prepare": (_i32, [_vp, _i32, _i32, _vp, _vp]),
    "moe_route": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _u32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_lru_reset": (_i32, [ctypes.POINTER(moe_lru), _vp]),
    "moe_lru_resize_workspace": (_sz, [_i32]),
    "moe_lru_resize": (_i32, [ctypes.POINTER(moe_lru), _vp, ctypes.POINTER(moe_lru), _vp, _sz, _sz, _vp, _sz,
                              _vp]),
    "moe_miss_record_words": (_sz, [_i32, _i32, _i32]),
    "moe_cache_lookup": (_i32, [ctypes.POINTER(moe_lru), _vp, _i32, _i32, _vp, _vp, _vp, _vp]),
    "moe_cache_fill": (_i32, [_vp, _vp, _vp, _sz, _sz, _vp, _vp, _vp]),
    "moe_ffn_workspace": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "moe_expert_ffn": (_i32, [_i32, _vp, _sz, _i32, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp,
                              _vp, _i32, _vp, _vp, _vp, _u32, _vp, _sz, _vp]),
    "moe_combine": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "moe_layer_workspace": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "moe_layer_forward": (_i32, [_i32, _vp, _sz, _i32, _i32, _i32, _i32, _u32, _vp, _i32, _vp, _vp, _vp,
                                 _vp, _vp, _sz, _vp]),
    "moe_layer_forward_prefetch": (_i32, [_i32, _vp, _sz, _i32, _i32, _i32, _i32, _u32, _vp, _i32, _vp, _vp,
                                          _vp, _vp, _vp, _sz, _vp, _sz, _vp]),
    "moe_layer_forward_static": (_i32, [_i32, _vp, _sz, _i32, _i32, _i32, _i32, _u32, _vp, _i32, _vp, _vp, _vp,
                                        _vp, _vp]),
    "moe_cached_layer_workspace": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "moe_cache_fill_device": (_i32, [_vp, _vp, _vp, _sz, _sz, _vp, _vp, _vp, _vp]),
    "moe_cached_layer_enqueue": (_i32, [_i32, _sz, _i32, _i32, _i32, _i32, _u32,
                                        ctypes.POINTER(moe_cached_layer), _vp, _i32, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _sz, _vp]),
    "moe_cached_layer_forward": (_i32, [_i32, _sz, _i32, _i32, _i32, _i32, _u32,
                                        ctypes.POINTER(moe_cached_layer), _vp, _i32, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _sz, _vp, _vp, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_int32)]),
    "moe_host_expert_ffn": (_i32, [_i32, _i32, _i32, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                   ctypes.POINTER(_vp), _vp, _i32]),
    "moe_cached_layer_split_host_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "moe_cached_layer_forward_split": (_i32, [_i32, _sz, _i32, _i32, _i32, _i32, _u32,
                                              ctypes.POINTER(moe_cached_layer), _vp, _i32, _vp, _vp, _vp, _vp,
                                              _vp, _vp, _sz, _vp, _vp, ctypes.c_float, _vp, _sz, _i32, _vp,
                                              ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                              ctypes.POINTER(ctypes.c_int32)]),
    "moe_prefetch_buffer_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "moe_prefetch_record_offset": (_sz, [_i32]),
    "moe_cached_layer_enqueue_prefetch": (_i32, [_i32, _sz, _i32, _i32, _i32, _i32, _u32,
                                                 ctypes.POINTER(moe_cached_layer), _vp, _i32, _vp, _vp, _vp, _vp,
                                                 _vp, _vp, _sz, _i32, _vp, _sz, _vp, _vp]),
    "moe_prefill_streamed_workspace": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "moe_prefill_streamed": (_i32, [_i32, _sz, _i32, _i32, _i32, _i32, _u32, _i32, ctypes.POINTER(_vp),
                                    ctypes.POINTER(_vp), _vp, _i32, ctypes.POINTER(_vp), _vp, _vp,
                                    ctypes.POINTER(_vp), _vp, _sz, _vp, _vp, ctypes.POINTER(_vp)]),
}

_lib = None


def lib():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: the HIP library must be built "
                               "(__graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        detail = lib().moe_last_error().decode()
        super().__init__(f"{where}: {lib().moe_status_str(status).decode()} ({status}) {detail}")


def _check(st, where):
    if st != MOE_OK:
        raise MoeError(st, where)


def _ptr(t):
    """Device/host address of a torch tensor or numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ blobs

def moe_expert_bytes(fmt, H, F):
    return int(lib().moe_expert_bytes(fmt, H, F))


def blob_stride(fmt, H, F):
    return (moe_expert_bytes(fmt, H, F) + 255) // 256 * 256


def _canon_ptrs(canon, fmt):
    keys = ("codes_g", "codes_u", "codes_d", "scales_g", "scales_u", "scales_d")
    arrs = [np.ascontiguousarray(canon[k]) for k in keys]
    taus = [np.array([canon.get("tau_" + m, 1.0)], dtype=np.float32) for m in "gud"]
    keep = arrs + taus
    ptrs = (_vp * 9)(*[a.ctypes.data for a in keep])
    return ptrs, keep


def moe_pack_expert(fmt, H, F, canon, blob=None):
    """Canonical dict -> packed blob (numpy uint8; written into ``blob`` if given)."""
    n = moe_expert_bytes(fmt, H, F)
    if blob is None:
        blob = np.empty(n, dtype=np.uint8)
    if blob.nbytes < n or not blob.flags["C_CONTIGUOUS"]:
        raise ValueError("blob too small or not contiguous")
    ptrs, keep = _canon_ptrs(canon, fmt)
    _check(lib().moe_pack_expert(fmt, H, F, ptrs, blob.ctypes.data), "moe_pack_expert")
    return blob


def moe_unpack_expert(fmt, H, F, blob):
    fp8 = fmt == MOE_FMT_FP8_E4M3
    cw = (lambda N, K: (N, K)) if fp8 else (lambda N, K: (N, K // 2))
    if fmt == MOE_FMT_NVFP4:
        sw, sdt = (lambda N, K: (N, K // 16)), np.uint8
    elif fmt == MOE_FMT_MXFP4:
        sw, sdt = (lambda N, K: (N, K // 32)), np.uint8
    else:
        sw, sdt = (lambda N, K: (N, K // 128)), np.float32
    out = dict(codes_g=np.empty(cw(F, H), np.uint8), codes_u=np.empty(cw(F, H), np.uint8),
               codes_d=np.empty(cw(H, F), np.uint8), scales_g=np.empty(sw(F, H), sdt),
               scales_u=np.empty(sw(F, H), sdt), scales_d=np.empty(sw(H, F), sdt))
    taus = [np.zeros(1, np.float32) for _ in range(3)]
    keys = ("codes_g", "codes_u", "codes_d", "scales_g", "scales_u", "scales_d")
    ptrs = (_vp * 9)(*([out[k].ctypes.data for k in keys] + [t.ctypes.data for t in taus]))
    blob = np.ascontiguousarray(blob)
    _check(lib().moe_unpack_expert(fmt, H, F, blob.ctypes.data, ptrs), "moe_unpack_expert")
    out["tau_g"], out["tau_u"], out["tau_d"] = (np.float32(t[0]) for t in taus)
    return out


def pack_layer(fmt, H, F, batch, dst, stride, threads=8):
    """Pack a synth ``experts`` batch (leading axis = expert) into ``dst`` at ``stride``.

    Experts are packed on a small thread pool (the C call releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    n = batch["codes_g"].shape[0]

    def one(i):
        canon = {k: batch[k][i] for k in ("codes_g", "codes_u", "codes_d", "scales_g", "scales_u", "scales_d")}
        canon["tau_g"], canon["tau_u"], canon["tau_d"] = batch["tau"][i]
        moe_pack_expert(fmt, H, F, canon, dst[i * stride:(i + 1) * stride])

    if threads <= 1 or n < 4:
        for i in range(n):
            one(i)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n)))
    return dst


# ---------------------------------------------------------------- routing

def moe_route_workspace(T, H, E, k):
    return int(lib().moe_route_workspace(T, H, E, k))


def new_route_workspace(T, H, E, k, device="cuda"):
    import torch
    return torch.empty(moe_route_workspace(T, H, E, k) + 256, dtype=torch.uint8, device=device)


class PreparedRouter:
    """A prepared router (moe_router_prepare): the fp32 router [E][H] then its
    three bf16 planes, in one uint8 device tensor `buf`.  Accepted wherever a
    router tensor is; the wrappers add MOE_ROUTE_PREPARED to the route flags.
    As a read-ahead buffer it stands for its fp32 part."""

    def __init__(self, router, stream=None):
        import torch
        self.E, self.H = (int(d) for d in router.shape)
        n = int(lib().moe_router_prepared_bytes(self.E, self.H))
        if n == 0:
            raise ValueError(f"moe_router_prepared_bytes({self.E}, {self.H}) = 0")
        self.buf = torch.empty(n + 256, dtype=torch.uint8, device=router.device)
        off = (-self.buf.data_ptr()) % 256
        self.buf = self.buf[off:off + n]
        r = router.contiguous()
        _check(lib().moe_router_prepare(_ptr(r), self.E, self.H, _ptr(self.buf), _stream(stream)),
               "moe_router_prepare")
        self.shape = (self.E, self.H)
        self.device = router.device

    def data_ptr(self):
        return self.buf.data_ptr()

    def numel(self):
        return self.E * self.H

    def element_size(self):
        return 4


def _route_flags(router, flags):
    return flags | MOE_ROUTE_PREPARED if isinstance(router, PreparedRouter) else flags


def moe_route(x, router, k, flags=0, topk_idx=None, topk_w=None, pair_perm=None, expert_off=None,
              ws=None, want_perm=True, stream=None):
    import torch
    T, H = x.shape
    E = router.shape[0]
    flags = _route_flags(router, flags)
    dev = x.device
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if want_perm and pair_perm is None:
        pair_perm = torch.empty(T * k, dtype=torch.int32, device=dev)
        expert_off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = new_route_workspace(T, H, E, k, dev)
    st = lib().moe_route(_ptr(x), _ptr(router), T, H, E, k, flags, _ptr(topk_idx), _ptr(topk_w),
                         _ptr(pair_perm), _ptr(expert_off), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_route")
    return topk_idx, topk_w, pair_perm, expert_off


# ------------------------------------------------------------------ cache

class LRUState:
    """LRU state in device memory (torch tensors) + the C struct view.  E is the
    number of keys; key_base the key of this view's expert 0 (views of one state
    with different key bases let several layers share one cache)."""

    key_base = 0

    def __init__(self, E, S, device="cuda", key_base=0):
        import torch
        self.E, self.S, self.key_base = E, S, key_base
        self.slot_expert = torch.full((S,), -1, dtype=torch.int32, device=device)
        self.expert_slot = torch.full((E,), -1, dtype=torch.int32, device=device)
        self.slot_stamp = torch.zeros(S, dtype=torch.int64, device=device)
        self.clock = torch.zeros(1, dtype=torch.int64, device=device)

    def view(self, key_base):
        """The same state (same tensors) seen from another key range."""
        v = LRUState.__new__(LRUState)
        v.__dict__.update(self.__dict__)
        v.key_base = key_base
        return v

    def c(self):
        return moe_lru(self.E, self.S, _ptr(self.slot_expert), _ptr(self.expert_slot),
                       _ptr(self.slot_stamp), _ptr(self.clock), self.key_base)


def moe_lru_reset(state, stream=None):
    s = state.c()
    _check(lib().moe_lru_reset(ctypes.byref(s), _stream(stream)), "moe_lru_reset")


def moe_lru_resize_workspace(S_new):
    return int(lib().moe_lru_resize_workspace(S_new))


def moe_lru_resize(src, src_pool, dst, dst_pool, expert_bytes, stride, ws=None, stream=None):
    """Resize a layer's slot cache from ``src`` (LRUState) to ``dst`` (LRUState with
    the new S; may share src's tensors) and move the kept blobs from ``src_pool``
    into ``dst_pool`` (the same tensor rebuilds the pool in place)."""
    import torch
    if ws is None:
        ws = torch.empty(moe_lru_resize_workspace(dst.S), dtype=torch.uint8, device=src.slot_expert.device)
    a, b = src.c(), dst.c()
    _check(lib().moe_lru_resize(ctypes.byref(a), _ptr(src_pool), ctypes.byref(b), _ptr(dst_pool), expert_bytes,
                                stride, _ptr(ws), ws.numel(), _stream(stream)), "moe_lru_resize")


def moe_miss_record_words(T, k, S):
    return int(lib().moe_miss_record_words(T, k, S))


def moe_cache_lookup(state, topk_idx, pair_slot, pair_order, miss_rec, stream=None):
    T, k = topk_idx.shape
    s = state.c()
    st = lib().moe_cache_lookup(ctypes.byref(s), _ptr(topk_idx), T, k, _ptr(pair_slot),
                                _ptr(pair_order), _ptr(miss_rec), _stream(stream))
    _check(st, "moe_cache_lookup")


def moe_cache_fill(miss_rec_host, host_pool, slot_pool, expert_bytes, stride, slots_free=None,
                   copy_stream=None, fill_done=None):
    ev = lambda e: None if e is None else e.cuda_event  # noqa: E731
    st = lib().moe_cache_fill(_ptr(miss_rec_host), _ptr(host_pool), _ptr(slot_pool), expert_bytes,
                              stride, ev(slots_free), _stream(copy_stream), ev(fill_done))
    _check(st, "moe_cache_fill")


# ------------------------------------------------------------ expert FFN

def moe_ffn_workspace(fmt, T, H, F, k, E):
    return int(lib().moe_ffn_workspace(fmt, T, H, F, k, E))


def new_ffn_workspace(fmt, T, H, F, k, E, device="cuda"):
    import torch
    return torch.empty(moe_ffn_workspace(fmt, T, H, F, k, E) + 256, dtype=torch.uint8, device=device)


def moe_expert_ffn(fmt, slot_pool, stride, H, F, E, x, topk_idx, pair_slot=None, pair_perm=None,
                   expert_off=None, pair_subset=None, topk_w=None, y=None, out=None, flags=0,
                   ws=None, stream=None):
    T, k = topk_idx.shape
    if ws is None:
        ws = new_ffn_workspace(fmt, T, H, F, k, E, x.device)
    n_subset = 0 if pair_subset is None else int(pair_subset.numel())
    st = lib().moe_expert_ffn(fmt, _ptr(slot_pool), stride, H, F, E, _ptr(x), T, k, _ptr(topk_idx),
                              _ptr(pair_slot), _ptr(pair_perm), _ptr(expert_off), _ptr(pair_subset),
                              n_subset, _ptr(topk_w), _ptr(y), _ptr(out), flags, _ptr(ws), ws.numel(),
                              _stream(stream))
    _check(st, "moe_expert_ffn")
    return y, out


def moe_combine(y, topk_w, out, stream=None):
    T, k = topk_w.shape
    H = y.shape[-1]
    _check(lib().moe_combine(_ptr(y), _ptr(topk_w), T, H, k, _ptr(out), _stream(stream)), "moe_combine")
    return out


# ------------------------------------------------------------ whole layer

def moe_layer_workspace(fmt, T, H, F, k, E):
    return int(lib().moe_layer_workspace(fmt, T, H, F, k, E))


def new_layer_workspace(fmt, T, H, F, k, E, device="cuda"):
    import torch
    return torch.empty(moe_layer_workspace(fmt, T, H, F, k, E) + 256, dtype=torch.uint8, device=device)


def moe_layer_forward(fmt, pool, stride, H, F, E, k, x, router, flags=0, topk_idx=None, topk_w=None,
                      out=None, ws=None, stream=None, warm=None):
    """moe_layer_forward; with `warm` (a device tensor, e.g. the next layer's
    router) moe_layer_forward_prefetch, which reads it ahead during the decode
    down kernel."""
    import torch
    T = x.shape[0]
    dev = x.device
    flags = _route_flags(router, flags)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.uint16, device=dev)
    if ws is None:
        ws = new_layer_workspace(fmt, T, H, F, k, E, dev)
    if warm is None:
        st = lib().moe_layer_forward(fmt, _ptr(pool), stride, H, F, E, k, flags, _ptr(x), T, _ptr(router),
                                     _ptr(topk_idx), _ptr(topk_w), _ptr(out), _ptr(ws), ws.numel(),
                                     _stream(stream))
        _check(st, "moe_layer_forward")
    else:
        st = lib().moe_layer_forward_prefetch(fmt, _ptr(pool), stride, H, F, E, k, flags, _ptr(x), T,
                                              _ptr(router), _ptr(topk_idx), _ptr(topk_w), _ptr(out), _ptr(ws),
                                              ws.numel(), _ptr(warm), warm.numel() * warm.element_size(),
                                              _stream(stream))
        _check(st, "moe_layer_forward_prefetch")
    return topk_idx, topk_w, out


# ----------------------------------------------------------- cached layer

def moe_cached_layer_workspace(fmt, T, H, F, k, E):
    return int(lib().moe_cached_layer_workspace(fmt, T, H, F, k, E))


class CachedLayer:
    """One layer's VRAM expert cache for moe_cached_layer_forward: router (device),
    host pool ([pinned] uint8 tensor of E blobs), slot pool (device, S blobs), LRU
    state, a pinned miss record and three events (created here)."""

    def __init__(self, router, host_pool, slot_pool, E, S, T, k, rec_on_device=False, lru=None):
        """lru: a shared LRUState view (keyed, e.g. ``state.view(j * E)`` for layer j
        of a group sharing one cache; slot_pool is then the group's pool)."""
        import torch
        self.router, self.host_pool, self.slot_pool = router, host_pool, slot_pool
        self.T, self.k, self.rec_on_device = T, k, rec_on_device
        if lru is None:
            self.lru = LRUState(E, S, router.device)
            moe_lru_reset(self.lru)
        else:
            self.lru = lru
        self._new_record()
        self.lookup_done, self.slots_free, self.fill_done = (torch.cuda.Event() for _ in range(3))
        for ev in (self.lookup_done, self.slots_free, self.fill_done):
            ev.record()  # creates the underlying HIP event
        torch.cuda.current_stream().synchronize()
        self._bind()

    def _new_record(self):
        import torch
        n = moe_miss_record_words(self.T, self.k, self.lru.S)
        self.miss_rec = (torch.zeros(n, dtype=torch.int32, device=self.router.device) if self.rec_on_device
                         else torch.zeros(n, dtype=torch.int32).pin_memory())

    def _bind(self):
        self.c = moe_cached_layer(_ptr(self.router), _ptr(self.host_pool), _ptr(self.slot_pool), self.lru.c(),
                                  _ptr(self.miss_rec), self.lookup_done.cuda_event, self.slots_free.cuda_event,
                                  self.fill_done.cuda_event)

    def resize(self, S_new, expert_bytes, stride, slot_pool=None, ws=None, stream=None):
        """Elastic resize to S_new slots (moe_lru_resize) between steps.  slot_pool=None
        rebuilds the current pool in place (it must hold S_new blobs); else the kept
        blobs move into the given pool, which the layer uses from then on."""
        pool = self.slot_pool if slot_pool is None else slot_pool
        if pool.numel() < S_new * stride:
            raise ValueError(f"slot pool holds {pool.numel() // stride} blobs < {S_new}")
        if slot_pool is None and S_new <= self.lru.S:   # the state shrinks inside its own tensors
            dst = LRUState.__new__(LRUState)
            dst.E, dst.S = self.lru.E, S_new
            dst.slot_expert, dst.slot_stamp = self.lru.slot_expert[:S_new], self.lru.slot_stamp[:S_new]
            dst.expert_slot, dst.clock = self.lru.expert_slot, self.lru.clock
            dst.key_base = self.lru.key_base
        else:
            dst = LRUState(self.lru.E, S_new, self.router.device, key_base=self.lru.key_base)
        moe_lru_resize(self.lru, self.slot_pool, dst, pool, expert_bytes, stride, ws=ws, stream=stream)
        self.lru, self.slot_pool = dst, pool
        if moe_miss_record_words(self.T, self.k, S_new) != self.miss_rec.numel():
            self._new_record()
        self._bind()


def moe_cached_layer_forward(fmt, stride, H, F, E, k, layer, x, topk_idx, topk_w, pair_slot, pair_order, out,
                             ws, flags=0, stream=None, copy_stream=None):
    """Returns (n_hits, n_miss) of the step; raises MoeError on MOE_E_CAPACITY."""
    if layer.rec_on_device:
        raise MoeError(MOE_E_ARG, "moe_cached_layer_forward reads the miss record on the host: "
                                  "the layer needs a pinned record (rec_on_device=False)")
    T = x.shape[0]
    hits, miss = ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib().moe_cached_layer_forward(fmt, stride, H, F, E, k, _route_flags(layer.router, flags), ctypes.byref(layer.c), _ptr(x), T,
                                        _ptr(topk_idx), _ptr(topk_w), _ptr(pair_slot), _ptr(pair_order),
                                        _ptr(out), _ptr(ws), ws.numel(), _stream(stream),
                                        _stream(copy_stream), ctypes.byref(hits), ctypes.byref(miss))
    _check(st, "moe_cached_layer_forward")
    return hits.value, miss.value


def new_split_host_workspace(T, H, F, k):
    import torch
    return torch.zeros(int(lib().moe_cached_layer_split_host_bytes(T, H, F, k)), dtype=torch.uint8).pin_memory()


def moe_cached_layer_forward_split(fmt, stride, H, F, E, k, layer, x, topk_idx, topk_w, pair_slot, pair_order, out,
                                   ws, q, host_ws, defer_done, threads=8, flags=0, stream=None, copy_stream=None):
    """The host-waiting cached layer with a share q of the misses computed on the
    CPU; returns (n_hits, n_miss, n_cpu)."""
    T = x.shape[0]
    if not defer_done.cuda_event:  # torch creates the HIP event at its first record
        defer_done.record()
    hits, miss, cpu = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib().moe_cached_layer_forward_split(fmt, stride, H, F, E, k, _route_flags(layer.router, flags), ctypes.byref(layer.c), _ptr(x), T,
                                              _ptr(topk_idx), _ptr(topk_w), _ptr(pair_slot), _ptr(pair_order),
                                              _ptr(out), _ptr(ws), ws.numel(), _stream(stream), _stream(copy_stream),
                                              float(q), _ptr(host_ws), host_ws.numel(), threads,
                                              defer_done.cuda_event, ctypes.byref(hits), ctypes.byref(miss),
                                              ctypes.byref(cpu))
    _check(st, "moe_cached_layer_forward_split")
    return hits.value, miss.value, cpu.value


def moe_cache_fill_device(miss_rec, host_pool, slot_pool, expert_bytes, stride, record_ready=None,
                          slots_free=None, copy_stream=None, fill_done=None):
    ev = lambda e: None if e is None else e.cuda_event  # noqa: E731
    st = lib().moe_cache_fill_device(_ptr(miss_rec), _ptr(host_pool), _ptr(slot_pool), expert_bytes, stride,
                                     ev(record_ready), ev(slots_free), _stream(copy_stream), ev(fill_done))
    _check(st, "moe_cache_fill_device")


def moe_cached_layer_enqueue(fmt, stride, H, F, E, k, layer, x, topk_idx, topk_w, pair_slot, pair_order, out,
                             ws, flags=0, stream=None):
    """Enqueue one cached layer on one stream (no host wait; misses streamed from the
    host pool); hits/misses are in layer.miss_rec once the stream has passed it."""
    T = x.shape[0]
    st = lib().moe_cached_layer_enqueue(fmt, stride, H, F, E, k, _route_flags(layer.router, flags), ctypes.byref(layer.c), _ptr(x), T,
                                        _ptr(topk_idx), _ptr(topk_w), _ptr(pair_slot), _ptr(pair_order),
                                        _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_cached_layer_enqueue")


def moe_host_expert_ffn(fmt, H, F, blobs, xs, threads=8):
    """Host expert FFNs: blobs (uint8 numpy/pinned arrays, one per pair), xs (bf16
    uint16 [H] rows) -> ys float32 [n, H]."""
    n = len(blobs)
    ys = np.zeros((n, H), np.float32)
    scratch = np.zeros(max(1, n * (H + F)), np.float32)
    xs = [np.ascontiguousarray(x, dtype=np.uint16) for x in xs]
    arr = lambda items: (_vp * max(1, n))(*[_ptr(a) for a in items])  # noqa: E731
    st = lib().moe_host_expert_ffn(fmt, H, F, n, arr(blobs), arr(xs), arr([ys[i] for i in range(n)]),
                                   _ptr(scratch), threads)
    _check(st, "moe_host_expert_ffn")
    return ys


def moe_prefetch_buffer_bytes(E, k, m, S):
    return int(lib().moe_prefetch_buffer_bytes(E, k, m, S))


def new_prefetch_buffer(E, k, m, S, device="cuda"):
    import torch
    return torch.zeros(moe_prefetch_buffer_bytes(E, k, m, S), dtype=torch.uint8, device=device)


def prefetch_record(pf_buf, E, k, m, S):
    """The prefetch step's miss record (a view of pf_buf)."""
    off = int(lib().moe_prefetch_record_offset(E))
    return pf_buf[off:off + 4 * moe_miss_record_words(1, k + m, S)].view(dtype=__import__("torch").int32)


def moe_cached_layer_enqueue_prefetch(fmt, stride, H, F, E, k, layer, x, topk_idx, topk_w, pair_slot, pair_order,
                                      out, ws, m, pf_buf, pf_stream, flags=0, stream=None):
    """moe_cached_layer_enqueue with the runner-up prefetch on pf_stream (T = 1)."""
    T = x.shape[0]
    st = lib().moe_cached_layer_enqueue_prefetch(fmt, stride, H, F, E, k, _route_flags(layer.router, flags), ctypes.byref(layer.c), _ptr(x), T,
                                                 _ptr(topk_idx), _ptr(topk_w), _ptr(pair_slot), _ptr(pair_order),
                                                 _ptr(out), _ptr(ws), ws.numel(), m, _ptr(pf_buf), pf_buf.numel(),
                                                 _stream(stream), _stream(pf_stream))
    _check(st, "moe_cached_layer_enqueue_prefetch")


# ------------------------------------------------- prefill with streamed experts

class PrefillStream:
    """Two VRAM pools of E blobs, a copy stream and the four events of
    moe_prefill_streamed (created here)."""

    def __init__(self, E, stride, device="cuda"):
        import torch
        self.pools = [torch.empty(E * stride, dtype=torch.uint8, device=device) for _ in range(2)]
        self.copy_stream = torch.cuda.Stream(device=device)
        self.events = [torch.cuda.Event() for _ in range(4)]
        for ev in self.events:
            ev.record()  # creates the underlying HIP event
        torch.cuda.current_stream().synchronize()


def moe_prefill_streamed_workspace(fmt, T, H, F, k, E):
    return int(lib().moe_prefill_streamed_workspace(fmt, T, H, F, k, E))


def moe_prefill_streamed(fmt, stride, H, F, E, k, host_pools, routers, x, outs, topk_idx, topk_w, ps, ws,
                         flags=0, stream=None):
    """Enqueue a prefill of x through len(host_pools) layers streamed from pinned host
    memory (ps: PrefillStream).  outs: list of bf16 [T][H]; topk_idx/topk_w: [L][T][k]."""
    L, T = len(host_pools), x.shape[0]
    arr = lambda xs: (_vp * max(1, len(xs)))(*[_ptr(t) for t in xs])  # noqa: E731
    evs = (_vp * 4)(*[e.cuda_event for e in ps.events])
    st = lib().moe_prefill_streamed(fmt, stride, H, F, E, k, _route_flags(routers[0], flags), L, arr(host_pools), arr(routers), _ptr(x), T,
                                    arr(outs), _ptr(topk_idx), _ptr(topk_w), arr(ps.pools), _ptr(ws), ws.numel(),
                                    _stream(stream), _stream(ps.copy_stream), evs)
    _check(st, "moe_prefill_streamed")
