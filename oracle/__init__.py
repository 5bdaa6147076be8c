"""CPU oracle for S2-Attn (LongLoRA's shift short attention).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's CPU
baseline leg may import this package; the library under
`shifted_sparse_attention_amd/` never does, and shares no code with it.

Plain numpy in float64, written from the method's description:
  * LongLoRA blog summary (smallflyingpig.github.io), section 3.3 "S^2-Attn":
    a length-L sequence is split into groups and attention runs inside each
    group; the worked shift example fixes the direction and size of the shift
    (half a group, towards earlier tokens).
  * nearauto.com article on LongLoRA, section on shift short attention: the
    method is two steps, shift the tokens of half the heads, then move groups
    from the token axis into the batch axis.
  * python88.com article, section on cutting the work into small pieces:
    heads are split in two and one half is shifted, so groups overlap.
  * LongLoRA blog, section 3.4: position interpolation squeezes positions
    [0, L) into [0, L0) for RoPE.

Two formulations are provided and tested against each other: the group form
(`s2attn.forward` / `s2attn.backward`: gather a group in rolled order, run
dense causal attention, scatter back) and the explicit-mask form
(`s2attn.forward_dense` / `s2attn.backward_dense`: an L x L mask, no rolling).
"""

from . import s2attn  # noqa: F401
