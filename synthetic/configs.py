"""The five synthetic workloads: model shapes, exploration sets, decoding mode,
prompt recipe and seeds.

They stand in for the trained checkpoints and evaluation datasets the DEX paper
uses (LayerSkip / Llama-2 / Qwen3 models on GSM8K, HumanEval and XSum, "Depth
Exploration for LLM Decoding", Section 4 and Appendix D), which are not
available here. All stages are uniform, as in the paper's DEX-1/K setting.

Conventions fixed here (inputs, not method arithmetic):
  * weights are N(0, 0.02) per element; the attention-output and FFN-down
    projections of layer l (1-based) are scaled by ``gamma ** l`` before the
    tensor is rounded to its storage dtype; norm weights are 1; no biases;
  * the LM head is tied to the embedding only where stated;
  * RoPE base 10000 and RMSNorm epsilon 1e-5 everywhere;
  * seeds: weights 1000+i, prompts 2000+i (2003 for the sampled 7B run), Gumbel
    3000+i, where i is the workload's ordinal.
"""

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    tied: bool
    dtype: str               # "f32" or "bf16": storage of weights and KV
    gamma: float             # residual-branch scale per layer
    X: Tuple[int, ...]       # exploration depths d_0 < ... < d_{N-1} = L
    batch: int
    mode: str                # "greedy" or "sample"
    tau: float
    prompt_len: int
    prompt_dist: str         # "uniform" or "zipf1.1"
    gen: int                 # new tokens per sequence
    seed_w: int
    seed_p: int
    seed_g: Optional[int]
    rope_base: float = 10000.0
    eps: float = 1e-5

    def scaled(self, **kw) -> "Workload":
        """A copy with some fields replaced (used for reduced-size test cases)."""
        return replace(self, **kw)


WORKLOADS = {
    # Tiny decoder, fp32, small enough for a CPU run in seconds.
    "tiny_f32": Workload(
        name="tiny_f32", n_layers=8, d_model=256, n_heads=4, n_kv_heads=4,
        head_dim=64, d_ffn=1024, vocab=2048, tied=True, dtype="f32",
        gamma=0.6, X=(2, 4, 6, 8), batch=1, mode="greedy", tau=1.0,
        prompt_len=32, prompt_dist="uniform", gen=64,
        seed_w=1001, seed_p=2001, seed_g=None),
    # Llama-2-7B-shaped, bf16, four exploration depths, greedy.
    "llama7b_x4_greedy": Workload(
        name="llama7b_x4_greedy", n_layers=32, d_model=4096, n_heads=32,
        n_kv_heads=32, head_dim=128, d_ffn=11008, vocab=32000, tied=False,
        dtype="bf16", gamma=0.85, X=(8, 16, 24, 32), batch=1, mode="greedy",
        tau=1.0, prompt_len=512, prompt_dist="uniform", gen=256,
        seed_w=1002, seed_p=2002, seed_g=None),
    # Same model, eight exploration depths, sampling at temperature 1.0.
    "llama7b_x8_sample": Workload(
        name="llama7b_x8_sample", n_layers=32, d_model=4096, n_heads=32,
        n_kv_heads=32, head_dim=128, d_ffn=11008, vocab=32000, tied=False,
        dtype="bf16", gamma=0.85, X=tuple(range(4, 33, 4)), batch=1,
        mode="sample", tau=1.0, prompt_len=1024, prompt_dist="uniform",
        gen=256, seed_w=1002, seed_p=2003, seed_g=3003),
    # Llama-2-13B-shaped, eight independent sequences, sampling at 0.7.
    "llama13b_x8_b8": Workload(
        name="llama13b_x8_b8", n_layers=40, d_model=5120, n_heads=40,
        n_kv_heads=40, head_dim=128, d_ffn=13824, vocab=32000, tied=False,
        dtype="bf16", gamma=0.88, X=tuple(range(5, 41, 5)), batch=8,
        mode="sample", tau=0.7, prompt_len=1024, prompt_dist="zipf1.1",
        gen=256, seed_w=1004, seed_p=2004, seed_g=3004),
    # Qwen3-8B-shaped grouped-query model (dimensions only), 16 sequences.
    "qwen8b_x9_b16": Workload(
        name="qwen8b_x9_b16", n_layers=36, d_model=4096, n_heads=32,
        n_kv_heads=8, head_dim=128, d_ffn=12288, vocab=151936, tied=False,
        dtype="bf16", gamma=0.9, X=tuple(range(4, 37, 4)), batch=16,
        mode="greedy", tau=1.0, prompt_len=8192, prompt_dist="uniform",
        gen=128, seed_w=1005, seed_p=2005, seed_g=None),
}

ORDER = ["tiny_f32", "llama7b_x4_greedy", "llama7b_x8_sample",
         "llama13b_x8_b8", "qwen8b_x9_b16"]


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]
