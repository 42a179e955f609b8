"""The five layer shapes this library is built and tested on.

The expert count and routing width of the large shapes (460 routed experts,
top-12) and the 8K token count come from the LightningLM 0.1V figures on the
skill card "Reversible Sparse MoE Single Node" (Architecture Details) and the
abstract of "Reversible Foundations: Training a 120B Sparse MoE through
State-Preserving Scaling".  Hidden sizes, adapter rank and quantisation group
are not given on those pages; the values below are this library's choices.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int          # mixes into the seed so every shape has its own streams
    T: int               # tokens
    d: int               # d_model
    E: int               # routed experts
    k: int               # experts per token
    f: int               # d_ff of each SwiGLU expert
    r: int               # adapter rank
    group: int           # int4 quantisation group along the reduction dim
    act: str             # "f32" or "bf16": activation / adapter storage dtype
    router_bias_var: float = 0.0   # 0 => no router bias
    lora_scale: float = 1.0
    train: bool = False  # forward + adapter-only backward
    bits: int = 4        # base storage: 4 (int4) or 8 (int8)

    @property
    def S(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


C1 = LayerConfig("tiny_f32", 1, T=64, d=128, E=8, k=2, f=256, r=4, group=32,
                 act="f32", train=True)
C2 = LayerConfig("bf16_e64", 2, T=4096, d=2048, E=64, k=6, f=1408, r=16,
                 group=128, act="bf16", train=True)
C3 = LayerConfig("bf16_e460_t8192", 3, T=8192, d=2048, E=460, k=12, f=768,
                 r=16, group=128, act="bf16", router_bias_var=0.5)
C4 = LayerConfig("decode_e460_t64", 4, T=64, d=2048, E=460, k=12, f=768, r=16,
                 group=128, act="bf16")
# Same seeded tensors as the 8K forward shape, plus the upstream gradient.
C5 = C3.with_(name="train_e460_t8192", train=True)

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5)}
