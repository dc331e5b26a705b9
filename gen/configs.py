"""The layer workloads: shapes, precision and the routing-skew recipe.

Shapes follow the DeepSeek-V3-style MoE layer described in the
Mixture-of-Kittens blog post ("Overlapping computation and communication in
MoE"): one shared expert plus many routed experts, top-k routing.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Dims:
    name: str
    T: int          # tokens
    d: int          # model dimension
    E: int          # routed experts
    k: int          # experts per token
    I: int          # routed-expert intermediate dimension
    S: int          # shared experts
    Is: int         # shared-expert intermediate dimension
    prec: str       # "f32", "bf16" or "mxfp8" (routed-expert GEMMs)
    zipf: float     # 0: no logit bias; else Zipf exponent of the expert-load skew
    backward: bool = False
    seed: int = 0

    @property
    def R(self):
        return self.T * self.k

    def fwd_flops(self):
        """Algorithmic forward FLOPs: router + routed SwiGLU FFNs + shared FFNs."""
        return (2 * self.T * self.d * self.E + 6 * self.T * self.k * self.d * self.I
                + 6 * self.T * self.S * self.d * self.Is)

    def bwd_flops(self):
        """Algorithmic backward FLOPs: three input-gradient and three
        weight-gradient GEMMs per FFN (twice the forward's), plus the router's
        weight and input gradients.  A recompute of the gate/up projections is
        not counted."""
        return (12 * self.T * self.k * self.d * self.I + 12 * self.T * self.S * self.d * self.Is
                + 4 * self.T * self.d * self.E)


CONFIGS = {
    "c0": Dims("c0", 256, 128, 8, 2, 64, 1, 64, "f32", 0.0),
    "c1": Dims("c1", 4096, 2048, 64, 6, 768, 1, 768, "bf16", 0.0),
    "c2": Dims("c2", 8192, 4096, 128, 8, 1536, 0, 0, "bf16", 0.0),
    "c3a": Dims("c3a", 8192, 7168, 256, 8, 2048, 1, 2048, "bf16", 1.2),
    "c3b": Dims("c3b", 32768, 7168, 256, 8, 2048, 1, 2048, "bf16", 1.2),
    "c4": Dims("c4", 16384, 7168, 256, 8, 2048, 1, 2048, "mxfp8", 1.2, backward=True),
}


# The layer shapes the Mixture-of-Kittens blog post benchmarks ("MoE layer
# benchmarks": experts, hidden size, expert intermediate size, top-k of the
# Kimi K2.7 Code, GLM-5.2, Qwen3.5-397B-A17B and DeepSeek-V4-Pro layers), as
# whole layers on one GPU at T=8192 (one shared expert of the routed
# intermediate size, the DeepSeek-V3-style layer the post targets; the
# router skew recipe of c3), and as one GPU's share of the post's runs (EP
# degree 64, 2,048 tokens per GPU before routing): the E/64 local experts and
# the 2,048·k rows they receive on average, each row routed to one local
# expert (k = 1 over the local experts, no skew, no shared expert: the shared
# expert runs on the source GPU's own 2,048 tokens).
SHAPES = {  # name: (E, d, I, k)
    "kimi_k27": (384, 7168, 2048, 8),
    "glm52": (256, 6144, 2048, 8),
    "qwen35": (512, 4096, 1024, 10),
    "dsv4pro": (384, 7168, 3072, 6),
    "dsv3": (256, 7168, 2048, 8),
}
for _n, (_E, _d, _I, _k) in SHAPES.items():
    if _n != "dsv3":
        CONFIGS[_n] = Dims(_n, 8192, _d, _E, _k, _I, 1, _I, "bf16", 1.2, backward=True)
        CONFIGS[_n + "_mx"] = Dims(_n + "_mx", 8192, _d, _E, _k, _I, 1, _I, "mxfp8", 1.2, backward=True)
    CONFIGS["ep64_" + _n] = Dims("ep64_" + _n, 2048 * _k, _d, _E // 64, 1, _I, 0, 0, "mxfp8", 0.0, backward=True)
N3 = [n for n in CONFIGS if n.split("_mx")[0] in SHAPES or n.startswith("ep64_")]


def get_config(name, **over):
    c = CONFIGS[name]
    if not over:
        return c
    fields = dict(c.__dict__)
    fields.update(over)
    return Dims(**fields)
