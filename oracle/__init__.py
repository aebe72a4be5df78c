"""CPU oracle for the fused NF4 QLoRA linear layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy implementation of what the HIP library computes: the NF4
codebook, blockwise absmax quantisation with double quantisation, dequantisation, and the QLoRA
layer Y = X deq(W)^T + s (X A^T) B^T with its backward dX, dA, dB, all products in float64, and
the gate/up pair of such layers joined by the SwiGLU activation (swiglu.py), the LoRA merge
W' = deq(W) + s B A (merge.py), the grouped mixture-of-experts layer (moe.py) and the 4-bit
floating-point (E2M1) variant of the weight format with FP8 group scales (fp4.py).

Only the test suite, the smoke check in __graft_entry__ and the CPU-baseline leg of bench.py may
import or run anything in this package. The product path (nf4_dequant_gemm_amd) never does: it
shares no code, table or constant with this package and fails loudly when its HIP library is
missing.

Sources. The method is named on the Unsloth pages (release article v0.1.463-beta, section "About
the Unsloth Project"; the Chinese v0.1.47-beta article, section on lowering the fine-tuning
barrier; the "Inside Unsloth" book listing, "What You'll Learn", "LoRA and QLoRA"): a frozen base
quantised to 4-bit NormalFloat with double quantisation of the quantisation constants, bf16 LoRA
adapters with Delta W = B A at rank r, and a fused dequant + matmul + LoRA launch that keeps
numerical equivalence. The pages give no level values, block size, rounding rule or nibble order;
the readings taken here are listed in nf4.py and qlora.py next to the code that takes them.

Parity status: every function here is pinned by tests/test_oracle_*.py against closed forms,
library routines (scipy's normal quantile, torch's bf16 conversion), brute force on tiny inputs,
exact identities (adjoints, linearity) and planted-mistake checks. No function is unpinned.
"""
from . import fp4, merge, moe, nf4, qlora, swiglu  # noqa: F401
