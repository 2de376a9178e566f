"""The workloads the path is measured and checked on.

Shapes follow one Qwen3-30B-A3B-style attention layer (Hq=32, Hkv=4, d=128);
selection settings follow the FlashPrefill V2 page's defaults (§4.1: block
B=128, 256 sink tokens, a 512-token window, alpha=0.1), i.e. 2 sink blocks
and 4 window blocks; the tiny case keeps 1 sink block and a 2-block window.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import synth


@dataclass(frozen=True)
class Workload:
    name: str
    lengths: tuple
    hq: int
    hkv: int
    d: int
    dtype: str              # "f32" | "bf16" | "e4m3"
    seed: int
    alpha: float
    sink_blocks: int
    window_blocks: int
    clusters: bool
    diag_bias: bool
    page_size: int = 0      # 0 = contiguous K/V
    q_lengths: tuple = None  # queries per request (the last positions); None = lengths

    def make(self):
        """Host batch (and the paged pool when page_size > 0)."""
        base_dtype = "bf16" if self.dtype == "e4m3" else self.dtype
        b = synth.make_batch(self.lengths, self.hq, self.hkv, self.d, self.seed, base_dtype,
                             clusters=self.clusters, diag_bias=self.diag_bias,
                             q_lengths=self.q_lengths)
        if self.dtype == "e4m3":
            b = synth.to_e4m3(b)
        paged = synth.page_kv(b, self.page_size, self.seed) if self.page_size else None
        return b, paged


TINY = Workload("tiny_2k_f32", (2048,), 4, 1, 128, "f32", 0, 0.1, 1, 2, False, False)
L32K = Workload("qwen3_30b_a3b_32k_bf16", (32768,), 32, 4, 128, "bf16", 1, 0.1, 2, 4, True, True)
L128K = Workload("qwen3_30b_a3b_128k_bf16", (131072,), 32, 4, 128, "bf16", 2, 0.1, 2, 4, True, True)
L128K_FP8 = Workload("qwen3_30b_a3b_128k_e4m3", (131072,), 32, 4, 128, "e4m3", 2, 0.1, 2, 4, True,
                     True)
VARLEN = Workload("paged_varlen_16req_bf16",
                  tuple(synth.varlen_lengths(16, 4096, 131072, 4)), 32, 4, 128, "bf16", 4, 0.1, 2,
                  4, True, True, page_size=64)

# Length sweep: 4 requests of equal length L, 4K..128K, same generator and
# selection settings as the 128K layer (one seed per length).
SWEEP = tuple(Workload(f"sweep_{L // 1024}k_x4_bf16", (L,) * 4, 32, 4, 128, "bf16", 100 + i, 0.1, 2, 4, True,
                       True) for i, L in enumerate((4096, 8192, 16384, 32768, 65536, 131072)))

# Chunked prefill ([V2] §4.3, Table 6): the queries of a request are the last
# chunk of its positions and the keys are everything before them as well.
# The last 8K and 16K chunks of a 128K prompt, a small fp32 case with an
# offset on no tile or block boundary, and a paged mix (one-query chunk, a
# fresh request, a request with no queries).
CHUNK_TINY = Workload("chunk_1000_of_3000_f32", (3000,), 4, 1, 128, "f32", 7, 0.1, 1, 2, False,
                      False, q_lengths=(1000,))
CHUNK_8K = Workload("chunk_8k_of_128k_bf16", (131072,), 32, 4, 128, "bf16", 2, 0.1, 2, 4, True,
                    True, q_lengths=(8192,))
CHUNK_16K = Workload("chunk_16k_of_128k_bf16", (131072,), 32, 4, 128, "bf16", 2, 0.1, 2, 4, True,
                     True, q_lengths=(16384,))
CHUNK_MIX = Workload("chunk_mix_paged_bf16", (20000, 9001, 65613, 3000, 7000), 32, 4, 128, "bf16", 9,
                     0.1, 2, 4, True, True, page_size=64, q_lengths=(8192, 9001, 8192, 1, 0))
CHUNKED = (CHUNK_TINY, CHUNK_8K, CHUNK_16K, CHUNK_MIX)

ALL = {w.name: w for w in (TINY, L32K, L128K, L128K_FP8, VARLEN) + SWEEP + CHUNKED}
