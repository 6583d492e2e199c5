"""The five workloads of the hot path, as data.

Sizes follow the DeepSeek-V4 description on the pages: CSA pools every 4 tokens
into one entry and HCA every 128 (botbeat.news, "Summary"; sameershanbhag.com,
"Two kinds of memory instead of one"), a sliding window keeps recent tokens
uncompressed, and contexts reach one million tokens.  The pages leave head
dims, top-k, indexer heads and gate details open; the values fixed here are the
ones the workloads below state.
"""
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Geometry:
    """Shapes shared by every layer of one workload."""
    H: int = 64            # query heads (all share one KV head)
    D: int = 512           # KV / query head dim
    D_r: int = 64          # trailing RoPE dims of D
    H_I: int = 64          # indexer heads
    d_I: int = 128         # indexer dim
    topk: int = 512        # entries kept per query
    n_win: int = 128       # sliding window, query token included
    m_csa: int = 4         # CSA compression ratio
    m_hca: int = 128       # HCA compression ratio
    tau: float = 1.0       # logit scale (queries carry 1/sqrt(D) already)
    rope_base: float = 10000.0

    @property
    def D_n(self) -> int:
        return self.D - self.D_r


TINY_GEOMETRY = Geometry(H=8, D=128, D_r=32, H_I=4, d_I=32, topk=16)
FULL_GEOMETRY = Geometry()


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    kind: str                 # tiny | csa_decode | hca_decode | csa_prefill | ragged_pair
    seed: int
    geometry: Geometry = FULL_GEOMETRY
    params: dict = field(default_factory=dict)
    description: str = ""

    def with_params(self, **kw):
        p = dict(self.params)
        p.update(kw)
        return replace(self, params=p)


CONFIGS = [
    WorkloadConfig(
        "tiny_f32", "tiny", 0, TINY_GEOMETRY,
        dict(L=2048, n_queries=16),
        "1 sequence, L=2048, D=128 (32 RoPE), 8 heads, CSA m=4 and HCA m=128 over one raw "
        "stream, indexer 4x32, top-16, window 128, sink 0, queries at 2032..2047, f32"),
    WorkloadConfig(
        "csa_decode_128k", "csa_decode", 1, FULL_GEOMETRY,
        dict(B=8, L=131072),
        "8 sequences x 131072 tokens, 64 heads, D=512 (448 FP8 + 64 BF16 RoPE), "
        "32768 CSA entries, FP8 indexer 64x128, top-512, window 128, per-head sink"),
    WorkloadConfig(
        "hca_decode_1m", "hca_decode", 2, FULL_GEOMETRY,
        dict(B=4, L=1048576),
        "4 sequences x 1048576 tokens, 8192 HCA entries each, dense shared-KV MQA, "
        "64 heads, D=512, window 128, per-head sink"),
    WorkloadConfig(
        "csa_prefill_1m", "csa_prefill", 3, FULL_GEOMETRY,
        dict(prefix=1048576, T=4096),
        "4096-token chunk after a 1048576-token prefix: pools 1024 CSA + 32 HCA entries, "
        "MXFP4 indexer 64x128 over 263168 keys, causal top-512, sparse MQA + window + sink"),
    WorkloadConfig(
        "ragged_pair_32", "ragged_pair", 4, FULL_GEOMETRY,
        dict(B=32, lo=4096, hi=1048576),
        "32 sequences, lengths log-uniform in [4096, 1048576], one CSA and one HCA decode "
        "layer per step, pool-on-completion"),
]


def config_by_name(name: str) -> WorkloadConfig:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
