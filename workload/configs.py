"""Workload shapes: one tiny cache-resident case and four model-shaped stacks.

The model shapes are those of the models the pages measure (OPT-30B,
Falcon-40B(ReLU) and LLaMA(ReGLU)-70B in the QbitAI article on r-manual.ru,
sections "Скорость вывода до 11 раз" and "Локальность вывода..."; Falcon 40B
and Llama 2 70B in the GeekNews summary, section "Đánh giá hiệu năng và demo",
including the INT4 runs).  The firing densities follow the pages' sparsity
figures (about 10% of OPT's FFN neurons fire; about 90% sparsity for the
sparsified models) and their power-law skew.  Real weights and prompts are
not used: every tensor is drawn from a seed.
"""

from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    d_model: int
    d_ff: int
    n_layers: int
    rank: int
    wtype: str            # "f32", "f16" or "q4_0" (FFN weights)
    act: str              # "relu", "reglu" or "relu2"
    rho: float            # mean firing probability
    zipf_s: float = 1.1
    w_std: float = 0.02
    tau: float = 0.5
    n_decode: int = 128   # decode tokens per layer
    batch: int = 1        # tokens per call in decode
    prompt: int = 0       # prompt length for the multi-token case (0: none)

    @property
    def pred_wtype(self) -> str:
        """Predictor weights stay fp16 when the FFN is Q4_0."""
        return "f16" if self.wtype == "q4_0" else self.wtype

    @property
    def x_dtype(self) -> str:
        """Activations are stored as the weights are; Q4_0 runs keep x in fp16."""
        return "f16" if self.wtype == "q4_0" else self.wtype

    @property
    def n_mat(self) -> int:
        return 3 if self.act == "reglu" else 2

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # Tiny ReLU FFN, fp32, one layer, eight decode tokens.
    "tiny": Config("tiny", 256, 1024, 1, 32, "f32", "relu", 0.15, n_decode=8),
    # OPT-30B-shaped ReLU stack, fp16, ~95% sparsity.
    "opt30b": Config("opt30b", 7168, 28672, 48, 1024, "f16", "relu", 0.05),
    # Falcon-40B(ReLU)-shaped stack, fp16, ~90% sparsity, plus a 64-token prompt.
    "falcon40b": Config("falcon40b", 8192, 32768, 60, 1024, "f16", "relu", 0.10, prompt=64),
    # Llama2-70B ReGLU-shaped stack (gate/up/down), predictor on the gate.
    "llama70b": Config("llama70b", 8192, 28672, 80, 1024, "f16", "reglu", 0.10),
    # Squared-ReLU variants (the pages list squared ReLU beside ReLU and ReGLU
    # as a supported activation): the tiny fp32 case and the Falcon shape.
    "tiny_relu2": Config("tiny_relu2", 256, 1024, 1, 32, "f32", "relu2", 0.15, n_decode=8),
    "falcon40b_relu2": Config("falcon40b_relu2", 8192, 32768, 60, 1024, "f16", "relu2", 0.10, prompt=64),
    # Q4_0 variants of the two large shapes, batch 1 and batch 8 decode.
    "falcon40b_q4": Config("falcon40b_q4", 8192, 32768, 60, 1024, "q4_0", "relu", 0.10),
    "llama70b_q4": Config("llama70b_q4", 8192, 28672, 80, 1024, "q4_0", "reglu", 0.10),
}


def get_config(name: str) -> Config:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None
