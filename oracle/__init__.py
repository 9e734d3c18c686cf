"""CPU oracle for the NF4 double-quantized QLoRA linear layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
reference written from the source pages.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The HIP library never calls, links or loads anything here, and
nothing here calls the HIP library: the two share no code, tables, constants
or helpers.

Page legend used in citations throughout this package:

* [P1] "QLoRA, in depth: when a 4-bit base is worth it for small language
  models, and how to ship the result" (aicassindra.com)
* [P2] "What is QLoRA, and how does 4-bit training make consumer-hardware
  fine-tuning possible?" (mantramindai.in)
* [P4] "QLoRA and Fine-Tuning on One Consumer GPU" (multigrid.ai)
* [P5] "QLoRA" (guide.dupenodi.dev)

Modules:

* :mod:`oracle.nf4_dq` -- NF4 table, block quantize, double quantize,
  dequantize, storage accounting.
* :mod:`oracle.qlora_linear` -- forward and backward of the adapted linear.
* :mod:`oracle.merge` -- merging the adapter into the weight and
  re-quantizing the result.
* :mod:`oracle.dropout` -- LoRA dropout of the adapter input: the
  counter-based mask generator and the dropped forward and backward.
* :mod:`oracle.formats` -- the storage-format variants the pages compare
  against (no double quantization; evenly spaced int4 levels).
* :mod:`oracle.f16` -- the fp16 compute-dtype instance (fp16 rounding and
  the fp16 dequant).

Every function pinned by a ``-m "not gpu"`` test says which pin covers it.
The one construction the pages leave fully open -- the tail offset of the
NF4 quantile grid -- is marked "parity unpinned" in :mod:`oracle.nf4_dq`.
"""

from .nf4_dq import (  # noqa: F401
    BLOCK,
    GROUP,
    TAIL_OFFSET,
    nf4_table_fp64,
    nf4_table,
    nf4_thresholds,
    bf16_bits_from_f32,
    f64_from_bf16_bits,
    block_absmax,
    nearest_codes,
    pack_codes,
    unpack_codes,
    double_quantize,
    quantize_nf4_dq,
    dequant,
    storage_bytes,
    bits_per_weight,
    quantize_groups,
)
from .qlora_linear import lora_scale, linear_fwd, linear_bwd, adapter_grads  # noqa: F401
from .merge import bf16_bits_from_f64, merge, requantize, requant_drift  # noqa: F401
from .dropout import (  # noqa: F401
    philox4x32_10,
    dropout_threshold,
    dropout_words,
    dropout_mask,
    linear_fwd_dropout,
    linear_bwd_dropout,
)
from . import formats  # noqa: F401
from . import f16  # noqa: F401
