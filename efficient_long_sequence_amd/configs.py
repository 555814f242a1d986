"""Workload table: the seven shapes the MiTA forward pass is checked and timed on.

Each workload names the shape of one batch of attention heads and the
synthetic value recipe (see :mod:`efficient_long_sequence_amd.synth`).  The
tiny fp32 case is sized so the CPU oracle finishes in well under a second; the
others follow the shapes the MiTA pages report on:

* DeiT-S on ImageNet-1K at 224x224 (14x14 patches, m = k = 25, s = 1;
  MiTA tutorial (iwxt.cn), ch.7, paper section 4.1 / Table 2);
* ADE20K segmentation at 512x512 and 640x640 (32x32 and 40x40 patches,
  m = k = 49, s = 1; same chapter, paper section 4.2 / Table 4);
* the long-sequence inference test with m*k = N/4 (same chapter, paper
  section 4.3 / Fig. 5), at N = 64K, 256K and 1M.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16"
    B: int
    H: int
    grid_h: int
    grid_w: int
    d: int
    land_h: int
    land_w: int
    k: int
    s: int
    kind: str           # "iid", "clustered", "runs"
    n_clusters: int
    seed: int

    @property
    def N(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def m(self) -> int:
        return self.land_h * self.land_w

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.N

    def with_s(self, s: int) -> "Workload":
        return replace(self, s=s, name=f"{self.name.split('_s')[0]}_s{s}")


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_n256_f32", "f32", 1, 1, 16, 16, 32, 4, 4, 16, 1, "iid", 0, 0),
        Workload("deit_s_n196", "bf16", 64, 6, 14, 14, 64, 5, 5, 25, 1, "clustered", 16, 1),
        Workload("ade_n1024", "bf16", 8, 6, 32, 32, 64, 7, 7, 49, 1, "clustered", 16, 2),
        Workload("ade_n1600", "bf16", 8, 6, 40, 40, 64, 7, 7, 49, 1, "clustered", 16, 3),
        Workload("long_n64k_s1", "bf16", 4, 2, 1, 65536, 64, 1, 128, 128, 1, "runs", 64, 4),
        Workload("long_n64k_s2", "bf16", 4, 2, 1, 65536, 64, 1, 128, 128, 2, "runs", 64, 4),
        Workload("long_n256k", "bf16", 1, 2, 1, 262144, 64, 1, 256, 256, 1, "runs", 256, 5),
        Workload("long_n1m", "bf16", 1, 2, 1, 1048576, 64, 1, 512, 512, 1, "runs", 256, 6),
    ]
}

# The long-sequence shapes the throughput metric is quoted on.
HEADLINE = "long_n1m"
LONG = ("long_n64k_s1", "long_n256k", "long_n1m")
