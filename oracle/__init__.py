"""Plain, slow CPU oracle for the NF4 QLoRA linear-layer path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``quantized_fine_tuning_amd``) never imports, links or executes anything here,
and nothing here imports the product path: the two share no code, no tables and
no constant generators.  The only module both sides use is ``workloads`` (seeded
input generators, which hold none of the method's arithmetic).

Everything here is written from the source pages, in numpy + the Python standard
library, in fp64 wherever the pages do not fix a precision.  Page tags used in
citations throughout:

  P1  "QLoRA 的原理是什么？4-bit 量化权重真的参与训练吗？"
      (offer.aigcbaba.com, fine-tuning / qlora-principle)
  P2  review of "QLoRA: Efficient Finetuning of Quantized LLMs"
      (www.ainexis.cn, papers / model-compression)
  P3  "Ch.09 QLoRA 与量化：缩得更小再微调" (mdooai.com, adv-dl / advDl09)
  P4  "M5 · PEFT (LoRA / QLoRA / Prefix Tuning)" science-depth card
      (airsota.com, 2026/10/01)
  P5  "Q103: What is QLoRA, and how does it differ from LoRA"
      (agentalpha.top, interview / finetune-tk409)

Modules:
  nf4        codebook, block absmax, nearest code, packing, e4m3, double
             quantization, dequantization, bf16 rounding
  linalg     fp64 forward / backward references of the QLoRA linear layer
  int8       the absmax INT8 scheme of P3 (used as a pin of the absmax
             convention)
  footprint  storage arithmetic (bits per parameter, bytes per tensor)
  adamw      the AdamW step on the LoRA parameters (fp32 states)
  merge      the LoRA adapter merged into the dequantized weight (16-bit
             output) and its re-quantization
  variants   comparison formats: NF4 without double quantization, absmax
             INT4 and INT8 (fp32 constant per 64-block)

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against something other than itself (page values, closed forms, brute force,
finite differences); none is "parity unpinned".
"""

from . import nf4, linalg, int8, footprint, adamw, merge, variants  # noqa: F401
