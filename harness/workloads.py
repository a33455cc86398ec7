"""Named synthetic workloads (shapes only) for tests and the benchmark.

The shapes are DeepSeek-V3/R1-style projection sizes: the pages' usage example
(DeepSeek DeepGEMM 中文讲解, "使用示例") uses M=4096, N=2112, K=7168; the rest
are the dense sweep, MoE grouped (contiguous and masked) and weight-gradient
shapes this library is measured on.  Seeds are SEED_BASE + workload index.
"""
from __future__ import annotations

from .inputs import SEED_BASE

# index 0: small dense case every tile/oracle path finishes in milliseconds
DENSE_SMALL = dict(name="dense_m128_n256_k512", m=128, n=256, k=512, seed=SEED_BASE + 0)

# index 1: dense sweep, M in {64,128,4096} x (N,K) pairs
DENSE_NK = [(2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168), (7168, 2048)]
DENSE_M = [64, 128, 4096]


def dense_sweep():
    out = []
    for m in DENSE_M:
        for (n, k) in DENSE_NK:
            out.append(dict(name=f"dense_m{m}_n{n}_k{k}", m=m, n=n, k=k, seed=SEED_BASE + 1))
    return out


# index 2: contiguous MoE, 8192 rows per expert, segment padding ~ U{0..127}
GROUPED_NK = [(4096, 7168), (7168, 2048)]


def contiguous_sweep():
    return [dict(name=f"contig_g{g}_n{n}_k{k}", g=g, rows_per_expert=8192, n=n, k=k,
                 seed=SEED_BASE + 2) for g in (4, 8) for (n, k) in GROUPED_NK]


# index 3: masked MoE decode, M_max = 256, masked_m ~ U{64..192}
def masked_sweep():
    return [dict(name=f"masked_g{g}_n{n}_k{k}", g=g, m_max=256, n=n, k=k,
                 seed=SEED_BASE + 3) for g in (1, 2, 4, 16) for (n, k) in GROUPED_NK]


# index 4: weight gradient dW[7168, 2048] over 4096 tokens, and the K-grouped
# variant over 4 experts with token counts {1024, 2048, 3072, 4096}
WGRAD = dict(name="wgrad_m7168_n2048_t4096", m=7168, n=2048, ks=[4096], seed=SEED_BASE + 4)
K_GROUPED_WGRAD = dict(name="kgrouped_wgrad_m7168_n2048_t1024_2048_3072_4096", m=7168, n=2048,
                       ks=[1024, 2048, 3072, 4096], seed=SEED_BASE + 4)
