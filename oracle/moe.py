"""The routed MoE layer forward, written out plainly in float64.

Gate ([753B] section "混合专家架构（MoE）的天然稀疏性"): a linear layer then a
softmax giving each expert's selection probability; the top-K experts are
evaluated and their outputs combined by a weighted sum.  Each expert is an
independent FFN.  Weights are dequantized at compute time ([8GB] §2.1); the
activations stay in bf16/fp64 (a stated reading: quantization is weight-only).

Per token t (x_t a bf16 row of width H; R the fp32 router [E, H]):
  1. z_t[e]  = fp32( sum_h x_t[h] * R[e,h] )           summed in fp64, rounded once
  2. p_t     = softmax(z_t) over all E experts          fp64 (softmax, then selection)
  3. S_t     = first k experts by (z desc, index asc)   (select on fp32 logits; ties
                                                          go to the lower index)
  4. w_tj    = fp32(p_t[S_tj]); with renorm, fp32(p_t[S_tj] / sum_j p_t[S_tj])
                                      (no renormalisation unless asked for)
  5. for each pair (t, j), e = S_tj, with G, U [F, H] and D [H, F] dequantized:
         g = G x_t,  u = U x_t                           fp64
         h = bf16( g / (1 + exp(-g)) * u )                one rounding; gate is the
                                                          first matrix, no bias/clamp
         y_tj = D h                                        fp64
  6. out_t = bf16( sum_{j=0..k-1} w_tj * y_tj )           fp64 sum in j order

Stacked layers are not chained: every layer of a step receives the same input
(a stated reading; chaining without norm or residual would shrink the
activations and carry rounding differences into later routing decisions).
"""

import numpy as np

from . import formats as fm


# ---------------------------------------------------------------------------
# router, softmax, top-k
# ---------------------------------------------------------------------------

def router_logits(x_bf16: np.ndarray, router: np.ndarray) -> np.ndarray:
    """Step 1: fp32 logits [T, E] from bf16 x [T, H] and fp32 router [E, H]."""
    x = fm.bf16_to_f64(x_bf16)
    r = np.asarray(router, dtype=np.float32).astype(np.float64)
    return fm.to_f32_rne(x @ r.T)


def softmax(z: np.ndarray) -> np.ndarray:
    """Step 2: softmax over the last axis in fp64 (shifted by the row max)."""
    z = np.asarray(z, dtype=np.float64)
    ez = np.exp(z - z.max(axis=-1, keepdims=True))
    return ez / ez.sum(axis=-1, keepdims=True)


def topk(z: np.ndarray, k: int) -> np.ndarray:
    """Step 3: per row, the k expert indices ordered by (logit desc, index asc).

    A stable sort of the negated logits keeps equal logits in ascending index
    order, which is the tie rule.  -0.0 and +0.0 compare equal.
    """
    z = np.asarray(z, dtype=np.float32)
    order = np.argsort(-z.astype(np.float64), axis=-1, kind="stable")
    return order[..., :k].astype(np.int32)


def route(x_bf16, router, k: int, renorm: bool = False):
    """Steps 1-4.  Returns (topk_idx int32 [T,k], topk_w float32 [T,k], logits)."""
    z = router_logits(x_bf16, router)
    p = softmax(z)
    idx = topk(z, k)
    psel = np.take_along_axis(p, idx.astype(np.int64), axis=-1)
    if renorm:
        psel = psel / psel.sum(axis=-1, keepdims=True)
    return idx, fm.to_f32_rne(psel), z


def top_margins(z: np.ndarray, k: int) -> np.ndarray:
    """Smallest gap between adjacent values among each row's k+1 largest logits.

    The generated-input rule asks this to be >= 1e-3 so that fp32 logits
    computed in a different summation order select the same experts.
    """
    z = np.sort(np.asarray(z, dtype=np.float64), axis=-1)[..., ::-1]
    kk = min(k + 1, z.shape[-1])
    top = z[..., :kk]
    if kk < 2:
        return np.full(z.shape[:-1], np.inf)
    return (top[..., :-1] - top[..., 1:]).min(axis=-1)


# ---------------------------------------------------------------------------
# experts
# ---------------------------------------------------------------------------

def dequant_expert(fmt: int, canon: dict):
    """Canonical expert bytes -> (G [F,H], U [F,H], D [H,F]) in float64.

    ``canon`` holds codes_g/u/d, scales_g/u/d and (NVFP4) tau_g/u/d.
    """
    mats = []
    for m in ("g", "u", "d"):
        tau = canon.get("tau_" + m, 1.0)
        mats.append(fm.dequant(fmt, canon["codes_" + m], canon["scales_" + m], tau))
    return tuple(mats)


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in fp64 (exp overflow gives -0 for g << 0)."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_ffn(G, U, D, x_rows_f64):
    """Step 5 for a batch of rows routed to one expert.

    Returns (h as float64 values of bf16, y float64 [m, H]).
    """
    g = x_rows_f64 @ G.T
    u = x_rows_f64 @ U.T
    h = fm.bf16_round_f64(silu(g) * u)
    y = h @ D.T
    return h, y


def combine(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Step 6: out[t] = bf16(sum_j w[t,j] * y[t,j,:]) summed in fp64 in j order."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    acc = np.zeros((y.shape[0], y.shape[2]), dtype=np.float64)
    for j in range(y.shape[1]):
        acc = acc + w[:, j:j + 1] * y[:, j, :]
    return fm.to_bf16_rne(acc)


def moe_layer(fmt: int, x_bf16, router, experts, k: int, renorm: bool = False,
              return_h: bool = False):
    """The whole layer for tokens x (bf16 [T, H]).

    ``experts`` maps an expert index to its canonical dict (a list, or any
    object with ``__getitem__``).  Only the routed experts are dequantized.
    Returns a dict with idx, w, logits, y (fp64 [T,k,H]) and out (bf16 [T,H]).
    """
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    T = x_bf16.shape[0]
    idx, w, z = route(x_bf16, router, k, renorm)
    xf = fm.bf16_to_f64(x_bf16)
    H = xf.shape[1]
    y = np.zeros((T, k, H), dtype=np.float64)
    hs = {}
    for e in np.unique(idx):
        G, U, D = dequant_expert(fmt, experts[int(e)])
        ts, js = np.nonzero(idx == e)
        h, ye = expert_ffn(G, U, D, xf[ts])
        y[ts, js] = ye
        if return_h:
            for n, (t, j) in enumerate(zip(ts, js)):
                hs[(int(t), int(j))] = h[n]
    res = dict(idx=idx, w=w, logits=z, y=y, out=combine(y, w))
    if return_h:
        res["h"] = hs
    return res


def dense_masked_layer(fmt: int, x_bf16, router, experts, E: int, k: int,
                       renorm: bool = False):
    """Pin for ``moe_layer``: evaluate EVERY expert on every token, then mix
    with a dense gate that is zero outside each token's top-k.

    Returns the fp64 pre-rounding mixture [T, H].  It must equal the sparse
    path's fp64 sum up to summation order.
    """
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    z = router_logits(x_bf16, router)
    p = softmax(z)
    T = z.shape[0]
    # dense mask by ranking every expert with a full sort (independent of topk())
    gate = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        ranked = sorted(range(E), key=lambda e: (-float(z[t, e]), e))
        chosen = ranked[:k]
        tot = sum(p[t, e] for e in chosen) if renorm else 1.0
        for e in chosen:
            gate[t, e] = float(np.float32(p[t, e] / tot))
    xf = fm.bf16_to_f64(x_bf16)
    acc = np.zeros((T, xf.shape[1]), dtype=np.float64)
    for e in range(E):
        G, U, D = dequant_expert(fmt, experts[e])
        _, ye = expert_ffn(G, U, D, xf)
        acc += gate[:, e:e + 1] * ye
    return acc


def combine_f64(y, w):
    """Pre-rounding fp64 value of ``combine`` (for pins)."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    acc = np.zeros((y.shape[0], y.shape[2]), dtype=np.float64)
    for j in range(y.shape[1]):
        acc = acc + w[:, j:j + 1] * y[:, j, :]
    return acc
