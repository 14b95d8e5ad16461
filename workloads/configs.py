"""The five synthetic workloads the hot path is checked and measured on.

Shapes follow the latent grids of the SANA-Video 2.0 pages (480p, 720p/5s and
720p/60s generation; 5B and 14B model widths; "SANA-Video 2.0" review page,
section 3, and the opennieuws news item, "Prestaties").  The pages give neither
head count nor head dimension; the values here (H = 24 or 40, d = 128) and the
token counts (latent frames x patch grid) are the workload definitions this
library is measured on, not quantities printed on the pages.
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                 # "f32" or "bf16": storage dtype of Q, K, V, G, O
    qkv_std: str               # "unit" (N(0,1)) or "rsqrt_d" (N(0,1)/sqrt(d))
    g_mean: float = 0.0        # G ~ N(g_mean, 1)
    heavy_frac: float = 0.0    # fraction of token rows of K and V scaled by heavy_scale
    heavy_scale: float = 4.0
    frames: int = 0
    grid: tuple = field(default=(0, 0))
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.B * self.N

    def tensor_bytes(self) -> int:
        return self.B * self.H * self.N * self.d * (4 if self.dtype == "f32" else 2)


CONFIGS = {
    # 4 latent frames x 8x8 patches; fp32 so the oracle runs in seconds.
    "tiny": Workload("tiny", 1, 2, 256, 64, "f32", "unit", frames=4, grid=(8, 8)),
    # 21 latent frames x 30x52 patches.
    "480p": Workload("480p", 1, 24, 32760, 128, "bf16", "rsqrt_d", frames=21, grid=(30, 52)),
    # 21 latent frames x 45x80 patches; the headline measurement shape.
    "720p5s": Workload("720p5s", 1, 24, 75600, 128, "bf16", "rsqrt_d", frames=21, grid=(45, 80)),
    # 241 latent frames x 45x80 patches, 5 % of K/V token rows scaled x4.
    "720p60s": Workload("720p60s", 1, 24, 867600, 128, "bf16", "rsqrt_d",
                        heavy_frac=0.05, frames=241, grid=(45, 80)),
    # 14B width: 40 heads, mostly-closed gates G ~ N(-1, 1).
    "14b": Workload("14b", 1, 40, 75600, 128, "bf16", "rsqrt_d", g_mean=-1.0,
                    frames=21, grid=(45, 80)),
    "14b_b2": Workload("14b_b2", 2, 40, 75600, 128, "bf16", "rsqrt_d", g_mean=-1.0,
                       frames=21, grid=(45, 80)),
}


def get(name: str) -> Workload:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None
