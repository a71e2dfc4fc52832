"""Seeded synthetic inputs for the paged KV-cache attention path.

This package is shared by the CPU oracle (``oracle/``) and by the HIP path
(``paged_kv_cache_67_amd``): both consume exactly the same arrays.  It draws
lengths, physical block placements and N(0,1) values, and nothing else: it
computes no slot addresses, no attention and no softmax, so that neither side
can inherit a mistake from it.

The workload shapes are those of the pages' models (Qwen2.5-0.5B and
Qwen3-0.6B attention layers, nano-vllm block size 256, mini-vLLM block size 16).
"""

from .synth import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_from_f32,
    make_config,
    make_mixed,
    make_tp_shard,
    make_workload,
    nan_bits,
    normal_values,
)
