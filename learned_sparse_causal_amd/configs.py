"""Workload shapes of the routed attention path.

Each entry fixes batch B, tokens T, width W, q/kv heads, head dim d, block size
beta, product code components P with K codes each (K**P addresses), list
capacity, minimum probes, R remote slots and L local blocks (the query's own
block included), and the activation dtype.  Weights are drawn N(0, 1/W) and
activations N(0, 1) by `synth`.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    T: int
    W: int
    Hq: int
    Hkv: int
    d: int
    beta: int
    P: int
    K: int
    cap: int
    n_probes: int
    R: int
    L: int
    dtype: str           # "f32" or "bf16"
    seed: int

    @property
    def NB(self):
        return self.T // self.beta

    @property
    def A(self):
        return self.K ** self.P

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def routes(self):
        return self.B * self.Hq * self.T

    def with_(self, **kw):
        return replace(self, **kw)

    def shape_kw(self):
        return dict(B=self.B, T=self.T, Hq=self.Hq, Hkv=self.Hkv, d=self.d, beta=self.beta,
                    P=self.P, K=self.K, cap=self.cap, n_probes=self.n_probes, R=self.R,
                    L=self.L)


# Tiny fp32: six blocks of 64 tokens, one local block, two remote slots (the
# technical report's associative-recall geometry: six blocks, five eligible
# at the latest queries, two selected).
TINY = Config("tiny_f32_T384", B=1, T=384, W=128, Hq=2, Hkv=2, d=64, beta=64, P=2, K=8,
              cap=8, n_probes=2, R=2, L=1, dtype="f32", seed=1001)

SMALL = Config("bf16_T4096", B=1, T=4096, W=512, Hq=8, Hkv=8, d=64, beta=64, P=2, K=16,
               cap=64, n_probes=4, R=2, L=2, dtype="bf16", seed=1002)

# All remote blocks eligible (R = NB - L), so every query bypasses the search
# and the result must equal dense causal attention.  Shape of a 360M-class
# model layer (width 960, 15 q heads / 5 kv heads, d 64).
ALL_ELIGIBLE = Config("all_eligible_T8192_gqa", B=1, T=8192, W=960, Hq=15, Hkv=5, d=64,
                      beta=64, P=2, K=16, cap=64, n_probes=4, R=127, L=1, dtype="bf16",
                      seed=1003)


def sweep(T):
    """Scaling sweep point: width 1024, 16 heads, 1024 addresses."""
    return Config("sweep_T%d" % T, B=1, T=T, W=1024, Hq=16, Hkv=16, d=64, beta=64, P=2, K=32,
                  cap=64, n_probes=4, R=2, L=2, dtype="bf16", seed=1004)


SWEEP_T = (4096, 8192, 16384, 32768)
SWEEP_32K = sweep(32768)

LARGE = Config("large_B8_T65536", B=8, T=65536, W=2048, Hq=16, Hkv=4, d=128, beta=128, P=2,
               K=32, cap=128, n_probes=8, R=8, L=2, dtype="bf16", seed=1005)

ALL = {c.name: c for c in (TINY, SMALL, ALL_ELIGIBLE, *(sweep(t) for t in SWEEP_T), LARGE)}
