"""CPU oracle for the routed block-scaled MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here.  The product
path (``block_scaled_fp4_gemv_amd``) never imports, links or calls this package,
and this package imports nothing from the product path: the two share no code.
The oracle takes the same canonical bytes the GPU path receives and computes,
slowly and plainly, in float64, what the layer is defined to compute.

Sources, cited throughout by key:

[753B]   Page "FreeToken：753B大模型塞进单卡的本地部署硬件账该怎么算" (kongchang.com).
         Section "混合专家架构（MoE）的天然稀疏性": each expert is an independent
         FFN; the gate is a linear layer followed by softmax that yields a
         selection probability per expert; the top-K experts are combined by a
         weighted sum.  Section "按带宽动态分配参数存储": routing-aware async
         copies on streams, frequency-based expert caching (LRU/LFU/ARC family).
[39TOK]  Page "8GB 笔记本 39.3 tok/s、单卡跑 753B：FreeToken 把 frontier MoE 拉回本地"
         (nxmr.cn).  Section "设计核心": a global LRU expert cache in VRAM absorbs
         routing locality of adjacent tokens; misses go to a "GPU cache fill".
         Section "局限": the system depends on NVFP4 / MXFP4 / FP8 weights.
[8GB]    Page "8GB显存跑35B MoE模型：FreeToken引擎本地部署实战" (xxmr.cn).
         §2.1: low-precision weights are dequantized to higher precision at
         compute time.  §2.2: only the routed experts are brought into VRAM.
[OCP-MX] OCP Microscaling Formats (MX) Specification v1.0: E2M1 elements, E8M0
         shared scale per 32 elements, scale exponent = floor(log2(amax)) - 2.
[OCP-F8] OCP 8-bit Floating Point Specification (OFP8): E4M3 "FN" variant,
         bias 7, no infinities, S.1111.111 is NaN, max finite 448.
[NVFP4]  NVIDIA's public NVFP4 description: E2M1 elements, one E4M3 scale per
         16 elements, and one fp32 per-tensor scale.

Everything not fixed by these sources is a stated reading (see the module
docstrings): softmax over all experts before selection, selection on fp32
logits with ties to the lowest expert index, no renormalisation by default,
SwiGLU = silu(gate) * up, bf16 rounding of the SwiGLU output and the layer
output only.
"""

from . import formats, moe, lru, permute  # noqa: F401
