"""The five workload shapes (sizes and fit parameters only, no arithmetic).

Each entry fixes a weight-matrix shape, the synthetic recipe that stands in
for real LLM weights and calibration activations, and the fit parameters:
sub-vector length d, codebook sizes and Lloyd iteration counts for the main
and residual stages, and the fraction of salient weights held exactly.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    cid: int            # seed component (1..5)
    name: str
    M: int              # output rows of W
    N: int              # input columns of W
    scale: float        # W = scale * StudentT(nu)
    nu: float
    bf16: bool          # W rounded to bfloat16 (round-to-nearest-even), held as fp32
    T: int              # calibration rows of X (T x N)
    n_ch: int           # high-energy activation channels
    ch_gain: float      # their multiplier
    d: int
    K1: int
    T1: int
    K2: int             # 0 = no residual stage
    T2: int
    p: float            # salient fraction held exactly
    binorm: bool

    @property
    def n_sub(self) -> int:
        return self.M * self.N // self.d


CONFIGS = [
    Config(1, "tiny-256x256", 256, 256, 0.02, 4.0, False, 128, 3, 20.0,
           8, 256, 10, 0, 0, 0.01, False),
    Config(2, "smollm2-proj-2048x2048", 2048, 2048, 0.02, 4.0, False, 512, 20, 20.0,
           8, 4096, 15, 256, 10, 0.005, False),
    Config(3, "mlp-up-8192x2048", 8192, 2048, 0.02, 3.0, False, 512, 20, 30.0,
           8, 65536, 10, 256, 10, 0.01, False),
    Config(4, "llama2-7b-mlp-4096x11008", 4096, 11008, 0.015, 4.0, True, 1024, 110, 20.0,
           8, 65536, 10, 256, 10, 0.01, True),
    Config(5, "70b-mlp-8192x28672", 8192, 28672, 0.01, 4.0, True, 1024, 286, 25.0,
           8, 65536, 8, 4096, 8, 0.01, False),
]

BY_NAME = {c.name: c for c in CONFIGS}


def get(cid_or_name):
    if isinstance(cid_or_name, int):
        return CONFIGS[cid_or_name - 1]
    return BY_NAME[cid_or_name]
