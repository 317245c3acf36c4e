"""The synthetic workloads: shapes, formats and distributions of the inputs.

Layer shapes follow the two model classes the FreeToken pages measure: a
35B-A3B-class MoE (hidden 2048, 256 experts, top-8, expert width 512, 40 MoE
layers) and a 753B-class MoE (hidden 6144, 256 experts, top-8, expert width
2048).  Values are synthetic: there are no trained weights.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    H: int
    E: int
    k: int
    F: int
    layers: int
    fmt: int                 # 1 NVFP4, 2 MXFP4, 3 FP8
    T: int                   # tokens per step (1 = batch-1 decode)
    steps: int
    w_std: float
    router_std: float = 0.05
    x_kind: str = "iid"      # "iid" bf16 N(0,1) rows, or "ar1" decode states
    slots: int = 0           # VRAM slots per layer (0 = all experts resident)
    fmts: tuple = field(default_factory=tuple)
    weights_cfg: int = -1    # seed group of the weights (-1 = cfg_id)

    @property
    def wcfg(self):
        return self.cfg_id if self.weights_cfg < 0 else self.weights_cfg

    @property
    def label(self):
        return self.name


WORKLOADS = {
    # tiny single layer, MXFP4, all resident
    "tiny": Workload("tiny", 0, H=256, E=8, k=2, F=512, layers=1, fmt=2, T=16, steps=1,
                     w_std=0.02),
    # 35B-A3B-like batch-1 decode, 40 stacked layers, NVFP4, AR(1) states
    "decode35b": Workload("decode35b", 1, H=2048, E=256, k=8, F=512, layers=40, fmt=1, T=1,
                          steps=256, w_std=0.02, x_kind="ar1"),
    # 35B-A3B-like prefill: 2048 tokens through one layer
    "prefill35b": Workload("prefill35b", 2, H=2048, E=256, k=8, F=512, layers=1, fmt=1, T=2048,
                           steps=1, w_std=0.02),
    # the same layer at 16384 tokens (512 rows per expert, about 1800 flop per
    # weight byte): a compute-bound point for the grouped MFMA kernels
    "prefill35b_16k": Workload("prefill35b_16k", 5, H=2048, E=256, k=8, F=512, layers=1, fmt=1,
                               T=16384, steps=1, w_std=0.02, weights_cfg=2),
    # cache-constrained decode: the decode35b layers (same weights), 64 of 256
    # experts per layer in VRAM, the rest in pinned host memory; own AR(1) states
    "cache35b": Workload("cache35b", 3, H=2048, E=256, k=8, F=512, layers=40, fmt=1, T=1,
                         steps=512, w_std=0.02, x_kind="ar1", slots=64, weights_cfg=1),
    # 753B-class layer stack: decode and 4096-token prefill, three formats
    "decode753b": Workload("decode753b", 4, H=6144, E=256, k=8, F=2048, layers=8, fmt=1, T=1,
                           steps=128, w_std=0.015, x_kind="ar1", fmts=(1, 2, 3)),
    "prefill753b": Workload("prefill753b", 4, H=6144, E=256, k=8, F=2048, layers=8, fmt=1,
                            T=4096, steps=1, w_std=0.015, fmts=(1, 2, 3)),
}
