"""Named workloads of response-replay attention.

Each preset fixes the shapes, dtypes, chunk and block partitions and the seed
of one synthetic workload.  The shapes follow the problem statement of
networkfinds.com/long-context-rl-is-a-state-lifetime-problem, section "Why
inference capacity does not imply training capacity" (a prompt of P tokens,
responses of lengths R_1..R_B) and the Qwen and GLM instantiations of
ai.thesatyajit.com/articles/longstraw-2m-rl, section "Two incompatible
architectures, same transaction" (GQA resident KV pages; MLA latent pages of
512 + 64 dims with DSA index keys).

This module holds sizes only: no arithmetic of the method.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    P: int                 # resident prompt positions
    R: int                 # response length (max over members for varlen)
    Hq: int                # query heads
    Hkv: int               # KV heads (1 for the latent variant)
    d_qk: int
    d_v: int
    chunk: int             # prompt chunk length (keys per softmax-statistics partial)
    block: int             # response block length of the reverse walk
    dtype: str             # "f32" or "bf16"
    seed: int
    G: int = 1             # responses replayed serially per group
    K: int = 1             # responses replayed concurrently (replay microbatch)
    r_min: Optional[int] = None   # varlen members: R_g uniform in [r_min, R]
    topk: int = 0          # 0 = dense; > 0 = per-query top-k prompt positions
    idx_dim: int = 0       # index-key width of the sparse selection
    latent: bool = False   # MLA latent pages: K = 576-wide latent row, V = its first d_v dims

    @property
    def tau(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    @property
    def n_chunks(self) -> int:
        return -(-self.P // self.chunk)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Tiny fp32 case, every element checked.
TINY_F32 = Workload("tiny_f32_P4096_R256", P=4096, R=256, Hq=4, Hkv=1, d_qk=64, d_v=64,
                    chunk=1024, block=256, dtype="f32", seed=1001)

# bf16 GQA with 8 KV heads.
GQA_P128K = Workload("bf16_gqa_P131072_R4096", P=131072, R=4096, Hq=32, Hkv=8, d_qk=128,
                     d_v=128, chunk=8192, block=2048, dtype="bf16", seed=1002)

# One context-parallel rank's share of a 2,097,152-position prompt (1/8).
SHARE_P256K = Workload("bf16_share_P262144_R8192", P=262144, R=8192, Hq=24, Hkv=4, d_qk=128,
                       d_v=128, chunk=16384, block=2048, dtype="bf16", seed=1003)

# Full 2,097,152-position resident prompt, G=8 serial members, R_g uniform in [2048, 8192].
FULL_P2M = Workload("bf16_full_P2097152_G8", P=2097152, R=8192, Hq=24, Hkv=4, d_qk=128,
                    d_v=128, chunk=32768, block=2048, dtype="bf16", seed=1004, G=8,
                    r_min=2048)

# Latent pages (512 + 64 rotary) shared by 64 heads, per-query top-2048 by fp32 index scores.
LATENT_P1M = Workload("bf16_latent_P1048576_R4096_top2048", P=1048576, R=4096, Hq=64, Hkv=1,
                      d_qk=576, d_v=512, chunk=65536, block=2048, dtype="bf16", seed=1005,
                      topk=2048, idx_dim=128, latent=True)

# LastKV chunk recurrence (zefan-cai.github.io/en/blog/lastkv-rl, section "LastKV: making
# recurrence boundaries part of the policy"): one layer's current chunk of R = 8192
# positions after P = 2,097,152 positions of history (256 completed chunks: last-layer K/V
# of the older ones, the blended previous chunk), the 2M configuration's heads.
LASTKV_P2M = Workload("bf16_lastkv_P2097152_C8192", P=2097152, R=8192, Hq=24, Hkv=4, d_qk=128,
                      d_v=128, chunk=32768, block=2048, dtype="bf16", seed=1006)

ALL = [TINY_F32, GQA_P128K, SHARE_P256K, FULL_P2M, LATENT_P1M, LASTKV_P2M]
BY_NAME = {w.name: w for w in ALL}


def flops_dense(Hq: int, d_qk: int, d_v: int, R: int, n_prompt_keys_per_row: int) -> dict:
    """Algorithmic flop count of one response's forward + response-only backward.

    Counted per visible (query row, key) pair and head: forward 2*d_qk (QK) + 2*d_v (PV);
    backward over prompt keys 2*d_qk (S recompute) + 2*d_v (dP) + 2*d_qk (dQ);
    backward over response keys additionally 2*d_qk (dK) + 2*d_v (dV).
    Masked pairs and the prompt dK/dV that the response-only contract never forms are
    not counted.
    """
    n_p = R * n_prompt_keys_per_row
    n_r = R * (R + 1) // 2
    fwd = Hq * (2 * d_qk + 2 * d_v) * (n_p + n_r)
    bwd = Hq * ((4 * d_qk + 2 * d_v) * n_p + (6 * d_qk + 4 * d_v) * n_r)
    return {"fwd": float(fwd), "bwd": float(bwd), "total": float(fwd + bwd),
            "prompt_pairs": n_p, "response_pairs": n_r}
