"""The five MoE-layer workloads, as data.

Shapes follow the expert-weight layouts of the Moebius review, §3.1 (weight
resharding): in the EP view a rank holds E/P whole experts with W13 of shape
(E/P, 2I, H) and W2 of shape (E/P, H, I); in the TP view it holds a slice of
every expert, W13 (E, 2I/P, H) and W2 (E, H, I/P).  The model shapes
(DeepSeek-V2-Lite, Qwen3-30B-A3B, Qwen3-235B-A22B) are the models the two pages
evaluate on.
"""
from dataclasses import dataclass, field
from typing import Tuple

POW2_BATCHES = (8, 16, 32, 64, 128, 256, 512, 1024, 2048)


@dataclass(frozen=True)
class LayerConfig:
    name: str
    H: int                 # hidden size
    E: int                 # routed experts in the gate
    k: int                 # routed experts per token
    renorm: bool           # renormalise the k picked probabilities to sum to 1
    I: int                 # full expert intermediate size
    dtype: str             # "fp32" or "bf16": storage type of x and weights
    T_list: Tuple[int, ...]
    routing: Tuple[str, ...] = ("uniform",)
    n_shared: int = 0      # always-on shared experts (weight 1, after routed)
    view: str = "full"     # "full", "ep" or "tp"
    P: int = 1             # ranks in the switch group (EP and TP views)
    description: str = ""

    @property
    def I_local(self) -> int:
        """Intermediate size held per expert by this GPU (I' = I, or I/P in TP)."""
        return self.I // self.P if self.view == "tp" else self.I

    @property
    def n_groups(self) -> int:
        """Expert groups whose weights this GPU holds."""
        if self.view == "ep":
            return self.E // self.P
        return self.E + self.n_shared

    @property
    def kk(self) -> int:
        """Columns of the routing table: k routed slots then the shared slots."""
        return self.k + self.n_shared

    @property
    def T_max(self) -> int:
        return max(self.T_list)

    def weight_bytes(self) -> int:
        s = 4 if self.dtype == "fp32" else 2
        return self.n_groups * 3 * self.H * self.I_local * s


CONFIGS = {
    "tiny": LayerConfig(
        name="tiny", H=256, E=8, k=2, renorm=True, I=128, dtype="fp32",
        T_list=(16,), routing=("uniform",),
        description="Tiny MoE layer, fp32: T=16, H=256, E=8, top-2 renormalised, I=128",
    ),
    "dsv2_lite": LayerConfig(
        name="dsv2_lite", H=2048, E=64, k=6, renorm=False, I=1408, dtype="bf16",
        T_list=(256,), routing=("uniform",), n_shared=2,
        description="DeepSeek-V2-Lite-shaped full layer: T=256, H=2048, 64 routed top-6 "
                    "(no renorm) + 2 shared experts, I=1408, bf16",
    ),
    "qwen3_30b": LayerConfig(
        name="qwen3_30b", H=2048, E=128, k=8, renorm=True, I=768, dtype="bf16",
        T_list=(8, 32, 128, 256, 1024, 2048), routing=("zipf", "uniform"),
        description="Qwen3-30B-A3B-shaped full layer: H=2048, E=128 top-8 renormalised, "
                    "I=768, bf16, log-Zipf(1.2) gate bias",
    ),
    "qwen3_235b_ep": LayerConfig(
        name="qwen3_235b_ep", H=4096, E=128, k=8, renorm=True, I=1536, dtype="bf16",
        T_list=POW2_BATCHES, routing=("uniform", "zipf"), view="ep", P=8,
        description="Qwen3-235B-A22B-shaped EP-rank share (P=8): 16 local experts, "
                    "W13 (16,3072,4096), W2 (16,4096,1536), bf16",
    ),
    "qwen3_235b_tp": LayerConfig(
        name="qwen3_235b_tp", H=4096, E=128, k=8, renorm=True, I=1536, dtype="bf16",
        T_list=POW2_BATCHES, routing=("uniform", "zipf"), view="tp", P=8,
        description="Qwen3-235B-A22B-shaped TP-rank share (P=8): all 128 experts sharded, "
                    "W13 (128,384,4096), W2 (128,4096,192), bf16, partial output",
    ),
}


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]
