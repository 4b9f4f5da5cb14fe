"""The five Hybrid Block workloads, as shapes and input-structure recipes.

Shapes follow the workload list that accompanies the HySparse2 pages; the
hyper-parameters k = 1024 global tokens and a 128-token local window come from
"Xiaomi Unveils HySparse2" (section "Token-Level Selection and Unified Local
Access") and from the bibibi.cc article (section "Article"), which also gives
the previous generation's 64-token groups.

A query chunk of n_q tokens sits at the end of its sequence: query i of a
sequence is at absolute position n_kv - n_q + i, and K/V already hold the
chunk's own tokens.
"""
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    cid: int                 # workload number 1..5 (0 = ad-hoc test shape)
    name: str
    dtype: str               # "fp32" or "bf16": Q, K, V and outputs
    batch: int
    n_q: int
    n_kv: int
    h_q: int
    h_kv: int
    d: int
    top_k: int = 1024
    window: int = 128
    n_sparse: int = 3        # sparse layers reusing the full layer's K/V and indices
    structure: str = "none"  # "none" | "needles" | "boost" | "clusters"
    extra: dict = field(default_factory=dict)
    block_size: int = 64     # block-selection ablation only
    top_blocks: int = 16

    @property
    def q_off(self) -> int:
        return self.n_kv - self.n_q

    @property
    def index_width(self) -> int:
        return self.top_k + self.window

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


CONFIGS = {
    1: Workload(1, "tiny_fp32_4k", "fp32", batch=1, n_q=4096, n_kv=4096,
                h_q=4, h_kv=1, d=64, n_sparse=3),
    2: Workload(2, "prefill_bf16_32k_needles", "bf16", batch=1, n_q=32768,
                n_kv=32768, h_q=32, h_kv=4, d=128, n_sparse=3,
                structure="needles", extra={"n_needles": 256, "needle_norm": 4.0}),
    3: Workload(3, "decode_bf16_64x128k", "bf16", batch=64, n_q=1, n_kv=131072,
                h_q=32, h_kv=4, d=128, n_sparse=3, structure="boost",
                extra={"boost_frac": 0.01, "boost_scale": 3.0}),
    4: Workload(4, "chunk_bf16_8k_on_262k", "bf16", batch=1, n_q=8192,
                n_kv=262144 + 8192, h_q=32, h_kv=4, d=128, n_sparse=5),
    5: Workload(5, "chunk_bf16_16k_on_1m", "bf16", batch=1, n_q=16384,
                n_kv=1048576, h_q=64, h_kv=8, d=128, n_sparse=7,
                structure="clusters",
                extra={"n_clusters": 32, "cluster_len": 32, "boost_scale": 3.0}),
}


def workload(cid_or_name) -> Workload:
    if isinstance(cid_or_name, Workload):
        return cid_or_name
    if isinstance(cid_or_name, int):
        return CONFIGS[cid_or_name]
    for w in CONFIGS.values():
        if w.name == cid_or_name:
            return w
    raise KeyError(cid_or_name)
