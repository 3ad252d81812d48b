"""Plain fp64 CPU oracle of the LatentMoE layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything under ``oracle/``: only the tests, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code, table or constant with the HIP library and does not import it.

Sources, cited by page title and section (the pages are web summaries of the
Nemotron 3 white paper and reports):
  [KO 2.2]   "NVIDIA Nemotron 3: Efficient and Open Intelligence 요약 설명"
             (greeksharifa.github.io), section 2.2 "LatentMoE: Hardware-Aware
             Expert Design for Improved Accuracy per Byte".
  [KO 2.4]   same page, section 2.4 "NVFP4 Training".
  [JA note]  "Nemotron 3: Efficient and Open Intelligence" wiki note
             (notes.yuuk.io), 提案手法 2 "LatentMoE".
  [Nano]     "Nemotron 3 Nano" blog post (jiwasawa.github.io), section on the
             granular Mixture-of-Experts, and its FP8 quantisation section.
  [Ultra]    "NVIDIA AI、Nemotron 3 Ultraをリリース" (news.chathome.org),
             architecture and quantization paragraphs.
Parity status of each function is stated in its docstring.
"""
from .moe import (  # noqa: F401
    E2M1_TABLE, E4M3_TABLE, OracleResult, bf16_to_f64, decode_expert, decode_nvfp4,
    e2m1_value, e4m3_qdq, e4m3_quantize, e4m3_value, expert_ffn, forward, forward_scalar, gates_softmax,
    latent_down, router_logits, route, select_top_k, sqrelu,
)
