"""CPU oracle for MLA absorbed decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and the
oracle imports nothing from the product path.  The two share only the seeded
input generator in ``workload/``, which holds no attention arithmetic.

Sources, cited by page title and section throughout (formula text on these
pages is partly garbled; each reading taken is stated where it is used):

* [V2 read-through] "DeepSeek-V2 paper" read-through, 2kiu.com/news/6085339 --
  section 2.1 (MHA cache accounting and the kv_cache_bytes script),
  2.3 (matrix absorption), 2.4 (decoupled RoPE), 5.1, 5.2, 6 (validation).
* [zeeklog] "Transformer 15: DeepSeek-V2 architecture (MLA, DeepSeekMoE)",
  zeeklog.com -- the MHA attention equation, equations 9-11, the cache table
  and the worked 576 / 32768 and 1/56 examples.
* [ai-library] "DeepSeek-V2" paper notes, process-cxr.github.io/ai-library --
  section "Multi-Head Latent Attention" (4.5 d_h l, shared k^R, concatenation).
* [V3 read-through] "DeepSeek-V3 technical report" read-through,
  2kiu.com/news/6340724 -- sections 2.2 (what is cached), 2.3 (absorption,
  k = [k_c; k_r]), 2.4, 4.1 (multi-token prediction used for speculative
  decoding, whose verification decodes several new tokens at once).

* [zeeklog] also: the YaRN paragraph (s = 40, alpha = 1, beta = 32, sqrt(t))
  and the d = 5120 hidden width of the worked example.
* [ai-library] also: "Model configuration" (RMSNorm after the compressed
  latent), "Long-Context Extension" (YaRN only on k^R) and "Training and
  Inference Efficiency" / "Inference cost" (the KV cache quantised to about 6
  bits per element at deployment).

Parity status: every function below is pinned by a test in
``tests/test_oracle_pins.py`` (decode), ``tests/test_oracle_append.py``
(cache append), ``tests/test_oracle_causal.py`` (several query tokens),
``tests/test_oracle_prefill.py`` (the unabsorbed chunk form) or
``tests/test_oracle_quant.py`` (low-bit cache) except where its docstring says
"parity unpinned".
"""

from .mla_ref import (  # noqa: F401
    absorb_query,
    cache_elems_per_token_mha,
    cache_elems_per_token_mla,
    default_scale,
    gather_rows,
    kv_cache_bytes,
    latent_attention,
    latent_attention_causal,
    mla_decode_absorbed,
    mla_decode_reference,
    mla_prefill_reference,
    project_out,
    softmax_attention,
    up_project,
)
from .quant_ref import (  # noqa: F401
    E4M3_MAX,
    dequantize_rows,
    e4m3_decode,
    e4m3_encode,
    quantize_rows,
)
from .append_ref import (  # noqa: F401
    append_into,
    append_rows,
    down_project,
    rms_norm,
    rope,
    rope_frequencies,
)
