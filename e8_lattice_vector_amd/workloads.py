"""Named cache shapes and codec settings of the pages' models.

Shapes: layers x KV heads x head_dim of Mistral-7B, Phi-3-mini, Llama-3.1-8B
and Qwen2.5-14B (NexusQuant blog, KV cache formula and memory-calculator
posts; Nedelkoski et al., Table 2).  Codec settings: K3V2 and K2V2 with a
scale per 64 or per head vector (nexusquant-kv 0.5.1 README, "How it works",
"Results"); theta per model family.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    S: int              # slabs = layers x batch
    H: int              # KV heads
    T: int              # tokens
    d: int              # head_dim
    theta: float        # RoPE base (0: none)
    bits_k: int
    bits_v: int
    G: int              # scale group (0: one per head vector)
    strict: bool
    fp32: bool = False
    with_v: bool = True
    Hq: int = 0         # query heads for scoring (0: no scoring)


TINY = Workload("tiny", 1, 1, 64, 8, 0.0, 2, 2, 8, True, fp32=True, with_v=False)
MISTRAL = Workload("mistral-7b", 32, 8, 2048, 128, 1e6, 3, 2, 64, False)
PHI3 = Workload("phi-3-mini", 32, 32, 4096, 96, 1e4, 2, 2, 0, True)
LLAMA = Workload("llama-3.1-8b-32k", 32, 8, 32768, 128, 5e5, 2, 2, 0, False)
QWEN_DECODE = Workload("qwen2.5-14b-decode-b16", 16 * 48, 8, 16384, 128, 5e5, 2, 2, 0,
                       False, with_v=False, Hq=40)

ALL = {w.name: w for w in (TINY, MISTRAL, PHI3, LLAMA, QWEN_DECODE)}
