"""Shared test utilities: seeded layers, margin-filtered inputs, tolerances.

Inputs come from the seeded generator; the routing margin rule uses the
oracle's fp32 logits (top-(k+1) adjacent gaps >= 1e-3, else the token's row or
the step's innovation is redrawn with attempt+1).
"""
import numpy as np

from block_scaled_fp4_gemv_amd import binding as B
from block_scaled_fp4_gemv_amd import synth as sy
from oracle import formats as fm
from oracle import moe

MARGIN = 1e-3
REL_L2 = 5e-3      # per output row
MAX_ABS = 2e-2     # per output row


class Layer:
    """One seeded layer.  eager=False generates experts only when first used."""

    def __init__(self, fmt, H, E, F, cfg, layer, w_std, seed=0, eager=True):
        self.fmt, self.H, self.E, self.F = fmt, H, E, F
        self.cfg, self.layer, self.w_std, self.seed = cfg, layer, w_std, seed
        self.router = sy.router(seed, cfg, layer, E, H)
        self.stride = B.blob_stride(fmt, H, F)
        self._cache = {}
        self.batch = None
        if eager:
            self.batch = sy.experts(fmt, seed, cfg, layer, 0, E, H, F, w_std)
            for e in range(E):
                self._cache[e] = sy.expert_view(self.batch, e)

    def expert(self, e):
        e = int(e)
        if e not in self._cache:
            b = sy.experts(self.fmt, self.seed, self.cfg, self.layer, e, 1, self.H, self.F, self.w_std)
            self._cache[e] = sy.expert_view(b, 0)
        return self._cache[e]

    @property
    def experts(self):
        layer = self

        class _View:
            def __getitem__(self, e):
                return layer.expert(e)
        return _View()

    def blob(self, e):
        return B.moe_pack_expert(self.fmt, self.H, self.F, self.expert(e))

    def host_pool(self, out=None):
        if out is None:
            out = np.empty(self.E * self.stride, np.uint8)
        if self.batch is not None:
            B.pack_layer(self.fmt, self.H, self.F, self.batch, out, self.stride)
        else:
            for e in range(self.E):
                n = B.moe_expert_bytes(self.fmt, self.H, self.F)
                B.moe_pack_expert(self.fmt, self.H, self.F, self.expert(e), out[e * self.stride:][:n])
        return out

    def device(self, needed=None):
        """(pool, router) on the GPU; with ``needed`` only those experts are filled."""
        import torch
        router = torch.from_numpy(np.ascontiguousarray(self.router)).cuda()
        if needed is None:
            return torch.from_numpy(self.host_pool()).cuda(), router
        pool = torch.zeros(self.E * self.stride, dtype=torch.uint8, device="cuda")
        for e in sorted(set(int(v) for v in np.asarray(needed).ravel())):
            b = torch.from_numpy(self.blob(e))
            pool[e * self.stride:e * self.stride + b.numel()].copy_(b)
        return pool, router


def margins_ok(x_bf16, routers, k):
    x = np.atleast_2d(x_bf16)
    ok = np.ones(x.shape[0], bool)
    for R in routers:
        ok &= moe.top_margins(moe.router_logits(x, R), k) >= MARGIN
    return ok


def iid_tokens(seed, cfg, T, H, routers, k, max_attempts=200):
    attempts = np.zeros(T, np.int64)
    x = sy.token_rows(seed, cfg, T, H)
    bad = ~margins_ok(x, routers, k)
    while bad.any():
        for t in np.nonzero(bad)[0]:
            attempts[t] += 1
            assert attempts[t] < max_attempts
            x[t] = sy.token_row(seed, cfg, int(t), H, int(attempts[t]))
        bad = ~margins_ok(x, routers, k)
    return x


def ar1_states(seed, cfg, n_steps, H, routers, k, max_attempts=200):
    out = np.empty((n_steps, H), np.uint16)
    a = 0
    h = sy.ar1_h0(seed, cfg, H)
    while not margins_ok(h, routers, k)[0]:
        a += 1
        assert a < max_attempts
        h = sy.normal_bf16(sy.stream(seed, cfg, sy.KIND_H0, 0, 0, 0, a), H)
    out[0] = h
    for t in range(1, n_steps):
        a = 0
        h = sy.ar1_next(out[t - 1], seed, cfg, t, H, a)
        while not margins_ok(h, routers, k)[0]:
            a += 1
            assert a < max_attempts
            h = sy.ar1_next(out[t - 1], seed, cfg, t, H, a)
        out[t] = h
    return out


def row_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = got - ref
    rl2 = np.linalg.norm(err, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    return rl2, np.abs(err).max(axis=-1)


def assert_rows_close(got, ref, rel=REL_L2, atol=MAX_ABS, what=""):
    rl2, mx = row_errors(got, ref)
    assert rl2.max() <= rel, f"{what}: rel-L2 {rl2.max():.3e} > {rel}"
    assert mx.max() <= atol, f"{what}: max-abs {mx.max():.3e} > {atol}"
    return rl2.max(), mx.max()


def bf16_dev_to_f64(t):
    return fm.bf16_to_f64(t.cpu().numpy().view(np.uint16))
