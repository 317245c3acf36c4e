"""Element and scale formats, decoded from their bit definitions, in float64.

E2M1 (FP4): bits S.EE.M, exponent bias 1, no inf/NaN; magnitudes
    0, 0.5, 1, 1.5, 2, 3, 4, 6 ([OCP-MX] element format; [NVFP4]).
E4M3 "FN": bits S.EEEE.MMM, bias 7; E=0 is subnormal m*2^-9; S.1111.111 is
    NaN; no infinities; max finite 448 ([OCP-F8]).
E8M0: unsigned exponent, value 2^(v-127); v=255 is NaN ([OCP-MX]).

Block-scaled weight tensors (the formats named in [39TOK] section "局限"), for a
matrix W of shape [N, K] whose blocks run along K (the reduction dimension) of
each output row (a stated reading; 16/32/128 divide every K used):
    NVFP4 : W[n,i] = e2m1(c[n,i]) * e4m3(s[n, i//16]) * tau           ([NVFP4])
    MXFP4 : W[n,i] = e2m1(c[n,i]) * 2^(s[n, i//32] - 127)            ([OCP-MX])
    FP8   : W[n,i] = e4m3(c[n,i]) * sigma[n, i//128]   (sigma fp32 per 128)

Canonical byte layout (the oracle's input):
    FP4 codes  uint8 [N, K/2], element 2i in the LOW nibble, 2i+1 in the high.
    FP8 codes  uint8 [N, K].
    NVFP4 scales uint8 [N, K/16];  MXFP4 scales uint8 [N, K/32];
    FP8 scales float32 [N, K/128];  NVFP4 tau: one float32 per matrix.

bf16 helpers: bf16 values travel as uint16 bit patterns.  ``to_bf16_rne``
rounds a float64 directly to bf16 (one rounding, ties to even).
"""

import numpy as np

NVFP4, MXFP4, FP8 = 1, 2, 3
FORMAT_NAMES = {NVFP4: "nvfp4", MXFP4: "mxfp4", FP8: "fp8"}
BLOCK = {NVFP4: 16, MXFP4: 32, FP8: 128}


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code from its sign, 2-bit exponent and 1-bit mantissa."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = m * 0.5  # subnormal: m * 2^(1-bias) * 2^-1
    else:
        mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3 (FN) code; NaN for S.1111.111."""
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        mag = m * 2.0 ** -9
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def e8m0_value(code: int) -> float:
    """Value of an E8M0 scale byte: 2^(code-127); NaN for 255."""
    if code == 255:
        return float("nan")
    return 2.0 ** (code - 127)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def unpack_fp4(codes: np.ndarray) -> np.ndarray:
    """uint8 [N, K/2] -> uint8 [N, K] of 4-bit codes (low nibble = even element)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0x0F
    out[..., 1::2] = codes >> 4
    return out


def _expand_blocks(scale_vals: np.ndarray, block: int) -> np.ndarray:
    return np.repeat(scale_vals, block, axis=-1)


def dequant_nvfp4(codes, scales, tau) -> np.ndarray:
    """NVFP4 matrix -> float64 [N, K] ([NVFP4]; tau is read as a dequant multiplier)."""
    v = E2M1_TABLE[unpack_fp4(codes)]
    s = E4M3_TABLE[np.asarray(scales, dtype=np.uint8)]
    return v * _expand_blocks(s, 16) * float(np.float32(tau))


def dequant_mxfp4(codes, scales) -> np.ndarray:
    """MXFP4 matrix -> float64 [N, K] ([OCP-MX])."""
    v = E2M1_TABLE[unpack_fp4(codes)]
    s = E8M0_TABLE[np.asarray(scales, dtype=np.uint8)]
    return v * _expand_blocks(s, 32)


def dequant_fp8(codes, scales) -> np.ndarray:
    """FP8 E4M3 matrix with an fp32 scale per 128 elements -> float64 [N, K]."""
    v = E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return v * _expand_blocks(s, 128)


def dequant(fmt: int, codes, scales, tau=1.0) -> np.ndarray:
    if fmt == NVFP4:
        return dequant_nvfp4(codes, scales, tau)
    if fmt == MXFP4:
        return dequant_mxfp4(codes, scales)
    if fmt == FP8:
        return dequant_fp8(codes, scales)
    raise ValueError(f"unknown format {fmt}")


# ----------------------------------------------------------------------------
# bf16
# ----------------------------------------------------------------------------

def bf16_to_f64(u16) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


_BF16_MIN_EXP = -126       # smallest normal exponent
_BF16_SUB_QUANTUM = 2.0 ** -133
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def to_bf16_rne(x) -> np.ndarray:
    """float64 -> bf16 bit patterns, one rounding to nearest, ties to even.

    A finite x is rounded to 8 significant bits (normal range) or to a multiple
    of 2^-133 (subnormal range); magnitudes at or beyond max + half an ulp become
    infinity; NaN becomes the canonical quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    ax = np.abs(x)
    finite = np.isfinite(x)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    normal = finite & (ax >= 2.0 ** _BF16_MIN_EXP)
    # normal: 8 significant bits -> m*2^8 rounded (np.rint is ties-to-even)
    out[normal] = np.ldexp(np.rint(np.ldexp(m[normal], 8)), e[normal] - 8)
    sub = finite & ~normal
    out[sub] = np.rint(x[sub] / _BF16_SUB_QUANTUM) * _BF16_SUB_QUANTUM
    out[~finite] = x[~finite]
    overflow = finite & (np.abs(out) > _BF16_MAX)
    out[overflow] = np.copysign(np.inf, x[overflow])
    f32 = out.astype(np.float32)            # exact: <= 8 significant bits
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    bits[np.isnan(x)] = 0x7FC0
    return bits


def bf16_round_f64(x) -> np.ndarray:
    """float64 -> the float64 value of its bf16 RNE rounding."""
    return bf16_to_f64(to_bf16_rne(x))


def to_f32_rne(x) -> np.ndarray:
    """float64 -> float32, IEEE round to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
