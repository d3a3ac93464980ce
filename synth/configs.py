"""The synthetic MoE layer shapes used for parity tests and measurement.

Shapes come from the models the pages name:
  * "tiny": a toy layer the CPU oracle evaluates in milliseconds.
  * "mt_encoder": the MoE FFN of the encoder-decoder MT model of "Who Says Elephants
    Can't Run" (section 3, model table: hidden 1024, FFN 4096, 32 experts, Switch top-1).
    T = 3840 stands for 96 sentences x 40 tokens (section 5: ~40K tokens in 1000
    sentences; batch 96 in the end-to-end throughput table).
  * "qwen15_moe", "dsv2_lite", "phi35_moe": the fine-grained expert shapes of the Specter
    page ("Technical novelty": 2048x1408 and 4096x6400 expert matrices; "Core method":
    speculation depths 16/8/16, batched verify B=32).

Only shapes, value distributions and seeds live here.
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int
    d: int               # hidden size (K of the first GEMM, N of the second)
    inter: int           # FFN width (ReLU) or SwiGLU intermediate size I
    E: int               # routed experts
    k: int               # experts per token
    act: str             # "relu" | "swiglu"
    wtypes: Tuple[str, ...]   # weight code types built for this layer: "int4" | "int8"
                              # (make_inputs also takes "fp16": unquantized experts)
    group: int           # 0 = per output channel, scales (E,1,N); 128 = groups along K
    gate_mode: str       # "topk" = softmax over the k chosen; "all" = softmax over all E
    zipf_bias: bool      # add the per-expert Zipf(1.1) log-bias to the logits
    T_list: Tuple[int, ...]
    n_shared: int = 0    # always-on fp16 shared experts (weight 1)
    shared_inter: int = 0
    sweep_active: Tuple[int, ...] = field(default_factory=tuple)

    @property
    def n1(self) -> int:
        """Columns of the first GEMM: F for ReLU, 2I ([gate | up]) for SwiGLU."""
        return 2 * self.inter if self.act == "swiglu" else self.inter


CONFIGS = {
    "tiny": LayerConfig("tiny", 1, d=128, inter=256, E=8, k=2, act="relu",
                        wtypes=("int4",), group=0, gate_mode="topk", zipf_bias=False,
                        T_list=(16,)),
    "mt_encoder": LayerConfig("mt_encoder", 2, d=1024, inter=4096, E=32, k=1, act="relu",
                              wtypes=("int4", "int8"), group=0, gate_mode="all",
                              zipf_bias=True, T_list=(3840,),
                              sweep_active=(1, 4, 8, 16, 24, 32)),
    "qwen15_moe": LayerConfig("qwen15_moe", 3, d=2048, inter=1408, E=60, k=4, act="swiglu",
                              wtypes=("int4",), group=128, gate_mode="topk", zipf_bias=True,
                              T_list=(17, 544)),
    "dsv2_lite": LayerConfig("dsv2_lite", 4, d=2048, inter=1408, E=64, k=6, act="swiglu",
                             wtypes=("int4",), group=128, gate_mode="all", zipf_bias=True,
                             T_list=(9, 288), n_shared=2, shared_inter=1408),
    "phi35_moe": LayerConfig("phi35_moe", 5, d=4096, inter=6400, E=16, k=2, act="swiglu",
                             wtypes=("int4",), group=128, gate_mode="topk", zipf_bias=False,
                             T_list=(1, 17, 8192)),
}


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]
