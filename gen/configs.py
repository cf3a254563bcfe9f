"""The five synthetic layer workloads (shapes and value distributions).

Shapes follow the routed-MoE layer the pages describe: 896 routed experts per
layer with 16 chosen per token and 2 always-on shared experts (kimi-k3-in-c
review, "at a glance" table; translated README, "shard census"), with the
hidden and intermediate sizes d = 7168 and f = 2048 of the workload definitions
this layer is measured on.  `tiny` is a shrunken layer with the same tensor
graph, small enough for pure-Python checks.
"""
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens
    d: int            # hidden size (contraction of router and gate/up)
    f: int            # routed expert intermediate size
    E: int            # routed experts
    k: int            # experts chosen per token
    n_shared: int     # always-on shared experts (bf16)
    f_shared: int     # shared expert intermediate size
    x_dtype: str      # 'f32' or 'bf16'
    out_dtype: str    # 'f32' or 'bf16'
    scale_lo: int     # E8M0 exponent range of routed weights, inclusive
    scale_hi: int
    router_sigma: float = 0.02
    shared_sigma: float = 0.02
    zipf_s: Optional[float] = None   # skewed routing through a bias channel
    seed: int = 0

    @property
    def P(self) -> int:
        return self.T * self.k

    def with_tokens(self, T: int, name: Optional[str] = None) -> "LayerConfig":
        d = dict(self.__dict__)
        d["T"] = T
        d["name"] = name or f"{self.name}_T{T}"
        return LayerConfig(**d)


_BIG = dict(d=7168, f=2048, E=896, k=16, n_shared=2, f_shared=2048, x_dtype="bf16",
            out_dtype="bf16", scale_lo=-10, scale_hi=-2)

CONFIGS = {
    "tiny": LayerConfig(name="tiny", T=4, d=256, f=128, E=16, k=4, n_shared=1, f_shared=128,
                        x_dtype="f32", out_dtype="f32", scale_lo=-8, scale_hi=0),
    "decode_b1": LayerConfig(name="decode_b1", T=1, **_BIG),
    "decode_b64": LayerConfig(name="decode_b64", T=64, **_BIG),
    "prefill_4096": LayerConfig(name="prefill_4096", T=4096, **_BIG),
    "prefill_16384_zipf": LayerConfig(name="prefill_16384_zipf", T=16384, zipf_s=1.1, **_BIG),
}

# Ordinal aliases in the order the workloads are listed.
ORDER = ["tiny", "decode_b1", "decode_b64", "prefill_4096", "prefill_16384_zipf"]


def get(name_or_index) -> LayerConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[ORDER[name_or_index]]
    return CONFIGS[name_or_index]
