"""The five synthetic workloads of the routed MoE layer.

Shapes follow the model the Strata pages describe: 512 routed experts per layer,
48 layers (24,576 experts), 10 active per token, shared experts beside the
routers ("Strata - the details", section "How it works"; the Strata README,
"How does it work?"). Decode runs over a speculative verify window of up to 4
tokens (3 MTP drafts + 1, "How it works"); prefill runs in chunks of 1,024 to
8,192 tokens ("Strata - the details", "Faster prompts"; v0.1.30 release notes,
"Faster short prompts").
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerConfig:
    cid: int            # workload id (0..4)
    name: str
    T: int              # tokens per layer step
    H: int              # hidden size
    E: int              # routed experts
    k: int              # experts per token
    I: int              # expert intermediate size
    shared: int         # 1 = one shared expert applied to every token with weight 1
    qtype: int          # 2 = Q2, 3 = Q3
    xdtype: str         # "f32" or "bf16" (activation and output dtype)
    zipf: bool          # per-expert Zipf(1.1) bias added to the router logits
    layers: int = 1     # independent layers of this shape
    streams: int = 1    # concurrent decode streams (tokens are streams x window)
    stream_ranking: bool = False  # each stream draws its own Zipf ranking of the experts

    @property
    def E_tot(self) -> int:
        return self.E + self.shared

    @property
    def A(self) -> int:
        """Expert assignments per layer step, shared expert included."""
        return self.T * (self.k + self.shared)

    def expert_bytes(self) -> int:
        """Packed bytes of one expert (gate, up, down), codes + (d, m) + high bits."""
        nb = 3 * self.H * self.I // 32
        per_block = 8 + 4 + (4 if self.qtype == 3 else 0)
        return nb * per_block

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS = {
    0: LayerConfig(0, "tiny", T=8, H=256, E=16, k=2, I=128, shared=0, qtype=2,
                   xdtype="f32", zipf=False),
    1: LayerConfig(1, "decode", T=4, H=2048, E=512, k=10, I=512, shared=1, qtype=2,
                   xdtype="bf16", zipf=True),
    2: LayerConfig(2, "prefill_1k", T=1024, H=2048, E=512, k=10, I=512, shared=1,
                   qtype=2, xdtype="bf16", zipf=True),
    3: LayerConfig(3, "prefill_8k_x48", T=8192, H=2048, E=512, k=10, I=512, shared=1,
                   qtype=2, xdtype="bf16", zipf=True, layers=48),
    4: LayerConfig(4, "batched_decode_q3", T=64, H=2048, E=512, k=10, I=512, shared=1,
                   qtype=3, xdtype="bf16", zipf=True, streams=16),
}


def get_config(cid: int) -> LayerConfig:
    return CONFIGS[int(cid)]
