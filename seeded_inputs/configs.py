"""The S2-Attn workloads, with their shapes, dtypes and seeds.

Shapes follow the Llama2 attention heads the LongLoRA pages fine-tune
(7B: 32 heads of d=128; 70B: 64 query heads sharing 8 KV heads), at the
contexts the pages extend to (model card, abstract: 7B to 100k, 70B to 32k).
The group size is a quarter of the context, the ratio under which the
nearauto.com article's Table 7 (ablations) attention FLOP shares come out.
Values are iid N(0, 1): the pages train on PG19 / RedPajama text, which is not
available here; dense unstructured draws stand in for the activations, and the
kernels' work does not depend on the values.

The first five are the S2-Attn training shapes; the two `causal` workloads
are the dense causal inference pass (one group spanning the whole context).
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    Hq: int
    Hkv: int
    d: int
    G: int
    shifted_heads: int
    dtype: str          # "f32" or "bf16": dtype of q, k, v, o, dO
    backward: bool      # whether the workload includes dQ, dK, dV
    seed: int
    rope: bool = False
    rope_base: float = 10000.0
    rope_orig_len: int = 4096
    note: str = field(default="", compare=False)

    @property
    def n_groups(self) -> int:
        return self.L // self.G

    @property
    def r(self) -> int:
        return self.Hq // self.Hkv

    def q_shape(self):
        return (self.B, self.L, self.Hq, self.d)

    def kv_shape(self):
        return (self.B, self.L, self.Hkv, self.d)


CONFIGS = {
    "fwd_f32_L256": Workload(
        name="fwd_f32_L256", B=1, L=256, Hq=4, Hkv=4, d=64, G=64,
        shifted_heads=2, dtype="f32", backward=False, seed=1,
        note="forward only, fp32; heads 2-3 rolled by G/2"),
    "fwd_bf16_L8k": Workload(
        name="fwd_bf16_L8k", B=1, L=8192, Hq=32, Hkv=32, d=128, G=2048,
        shifted_heads=16, dtype="bf16", backward=False, seed=2,
        note="forward, Llama2-7B attention shape"),
    "fwdbwd_bf16_L32k": Workload(
        name="fwdbwd_bf16_L32k", B=1, L=32768, Hq=32, Hkv=32, d=128, G=8192,
        shifted_heads=16, dtype="bf16", backward=True, seed=3,
        note="forward+backward, Llama2-7B heads at 32k context"),
    "fwdbwd_bf16_L100k_rope": Workload(
        name="fwdbwd_bf16_L100k_rope", B=1, L=102400, Hq=32, Hkv=32, d=128, G=25600,
        shifted_heads=16, dtype="bf16", backward=True, seed=4, rope=True,
        note="forward+backward, 100k context, RoPE with position interpolation to 4096"),
    "fwdbwd_bf16_L32k_gqa": Workload(
        name="fwdbwd_bf16_L32k_gqa", B=1, L=32768, Hq=64, Hkv=8, d=128, G=8192,
        shifted_heads=32, dtype="bf16", backward=True, seed=5,
        note="forward+backward, Llama2-70B grouped-query shape"),
    # Dense causal attention (G = L, no shifted heads): the inference pass the
    # pages run after fine-tuning, where S2-Attn is no longer used.
    "fwd_bf16_causal_L32k": Workload(
        name="fwd_bf16_causal_L32k", B=1, L=32768, Hq=32, Hkv=32, d=128, G=32768,
        shifted_heads=0, dtype="bf16", backward=False, seed=6,
        note="forward only, full causal attention over 32k tokens (inference)"),
    "fwd_bf16_causal_L100k": Workload(
        name="fwd_bf16_causal_L100k", B=1, L=102400, Hq=32, Hkv=32, d=128, G=102400,
        shifted_heads=0, dtype="bf16", backward=False, seed=7,
        note="forward only, full causal attention over 100k tokens (inference)"),
}

@dataclass(frozen=True)
class BlockWorkload:
    """One Llama-style attention block around S2-Attn with LoRA on Q, K, V, O."""
    name: str
    B: int
    L: int
    Hq: int
    Hkv: int
    d: int
    G: int
    shifted_heads: int
    lora_rank: int
    lora_scale: float
    seed: int
    rope: bool = False
    rope_base: float = 10000.0
    rope_orig_len: int = 4096
    note: str = field(default="", compare=False)

    @property
    def Dm(self) -> int:
        return self.Hq * self.d


BLOCK_CONFIGS = {
    "block_bf16_L1k": BlockWorkload(
        name="block_bf16_L1k", B=1, L=1024, Hq=4, Hkv=2, d=128, G=256, shifted_heads=2,
        lora_rank=8, lora_scale=2.0, seed=11, rope=True, rope_orig_len=256,
        note="small block: GQA, RoPE position interpolation 256 -> 1024"),
    "block_bf16_L8k": BlockWorkload(
        name="block_bf16_L8k", B=1, L=8192, Hq=32, Hkv=32, d=128, G=2048, shifted_heads=16,
        lora_rank=8, lora_scale=2.0, seed=13, rope=True, rope_orig_len=4096,
        note="Llama2-7B attention block at 8k (groups of L/4), RoPE position interpolation 4k -> 8k"),
    "block_bf16_L32k": BlockWorkload(
        name="block_bf16_L32k", B=1, L=32768, Hq=32, Hkv=32, d=128, G=8192, shifted_heads=16,
        lora_rank=8, lora_scale=2.0, seed=12, rope=True, rope_orig_len=4096,
        note="Llama2-7B attention block at 32k, RoPE position interpolation 4k -> 32k"),
}

# The workload the headline throughput is quoted on: fwd+bwd, Llama2-7B heads, L=32k.
HEADLINE = "fwdbwd_bf16_L32k"


def workload(name: str) -> Workload:
    return CONFIGS[name]
