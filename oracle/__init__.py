"""CPU oracle for DuoAttention's mixed retrieval/streaming attention.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plainly written fp64
definition that the GPU library is checked against.  Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it; the
library itself (``kv_cache_duo_amd``) never does, and this package imports
nothing from the library.  The two share no code.

Sources (the DuoAttention paper, arXiv 2410.10819, as described on the web
pages this project was built from):

* Abstract, as reproduced on the pith.science review page ("read the original
  abstract"): retrieval heads attend to every token; streaming heads attend
  to recent tokens and attention sinks and keep a constant-length cache.
* sourcepulse.org project card, "How It Works": full KV cache only for
  retrieval heads, a lightweight constant-length cache for streaming heads.
* pith.science referee report, minor comment 3: the pages give no equation
  for the cache size or for sink handling, so those steps follow the readings
  listed in ``mixed_attention`` and ``cache_state``.

Every function here is pinned by ``tests/test_oracle.py`` and
``tests/test_oracle_quant.py``, ``tests/test_oracle_rope.py`` and ``tests/test_oracle_fp8.py`` against closed forms, a library routine (torch
fp64 scaled-dot-product attention), brute force on tiny inputs and
hand-derived fixtures under ``tests/golden/``.  ``quantized_cache`` adds the
int8 retrieval cache the pages allude to ("combined with quantization",
abstract), with the scheme taken as a stated reading, and ``fp8_cache`` the
e4m3 alternative; ``rope`` adds rotary
position embedding on the way into the cache (cited by the pages only, in the
pith.science reference list), restated from its published definition.
"""

from .mixed_attention import (  # noqa: F401
    allowed_positions,
    attention_weights_row,
    attend_rows,
    mixed_attention,
)
from .cache_state import (  # noqa: F401
    CacheSimulator,
    streaming_slot_of_position,
    streaming_slot_positions,
)
from .quantized_cache import (  # noqa: F401
    dequantize_rows,
    quantize_rows,
    seen_rows,
)
from .rope import (  # noqa: F401
    apply_rope,
    rope_frequencies,
    rotated_qk,
    round_bf16,
)
from .fp8_cache import (  # noqa: F401
    dequantize_rows_fp8,
    e4m3_decode,
    e4m3_encode,
    quantize_rows_fp8,
    seen_rows_fp8,
)
