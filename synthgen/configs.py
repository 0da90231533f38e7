"""The five synthetic workloads, with the shapes the pages give.

Qwen-shaped (NVFP4: e2m1 codes, one E4M3 scale per 16 codes): hidden 2560,
expert intermediate 640, 512 experts, top-10, 48 MoE layers, one bf16 shared
expert per layer ([Q] "Why this model, of all models"; [Q] "The engine" items
1, 4, 5; 2451-token prompt from [Q] "The engine" item 5).

DeepSeek-shaped (MXFP4: e2m1 codes, one UE8M0 scale per 32 codes): hidden
4096, intermediate 2880, 384 experts, top-6 ([D] "Bytes per token decide
everything": 17.93 MiB per expert; [D] "Making it faster": 311-token prompt).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # experts per layer
    k: int            # experts per token
    fmt: str          # "nvfp4" | "mxfp4"
    layers: int       # MoE layers resident
    T: int            # tokens (decode: 1)
    shared: bool      # one bf16 shared expert per layer
    routing: str      # "router" (fp32 router GEMV) | "zipf" | "uniform" (drawn directly)
    zipf_s: float
    scale_lo: int     # scale bytes uniform over scale_lo..scale_hi
    scale_hi: int
    out_bf16: bool    # prefill output dtype

    @property
    def group(self) -> int:
        return 16 if self.fmt == "nvfp4" else 32

    @property
    def block_bytes(self) -> int:
        n = 3 * self.H * self.I
        return n // 2 + n // self.group

    @property
    def is_prefill(self) -> bool:
        return self.T > 1


# E4M3 codes 0x18..0x48 are the 49 contiguous codes from 2^-4 to 2^2.
# UE8M0 codes 121..129 are the exponents -6..2.
WORKLOADS = {
    "qwen_layer_decode": Workload("qwen_layer_decode", 1, 2560, 640, 64, 10, "nvfp4", 1, 1, False,
                                  "router", 0.0, 0x18, 0x48, False),
    "qwen_decode": Workload("qwen_decode", 2, 2560, 640, 512, 10, "nvfp4", 48, 1, True,
                            "router", 0.0, 0x18, 0x48, False),
    "qwen_prefill": Workload("qwen_prefill", 3, 2560, 640, 512, 10, "nvfp4", 1, 2451, False,
                             "zipf", 1.1, 0x18, 0x48, False),
    "deepseek_decode": Workload("deepseek_decode", 4, 4096, 2880, 384, 6, "mxfp4", 8, 1, False,
                                "router", 0.0, 121, 129, False),
    "deepseek_prefill": Workload("deepseek_prefill", 5, 4096, 2880, 384, 6, "mxfp4", 1, 311, False,
                                 "uniform", 0.0, 121, 129, True),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]
