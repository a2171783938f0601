"""CPU oracle for the hybrid sliding-window / INT8 / block-sparse attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``hybrid_swa_kv_amd``) never imports it, and this package imports
nothing from the product path: the two share no kernels, headers, helpers,
tables or constants.

Everything here is plain and slow on purpose: numpy, fp64 for attention and
block selection, IEEE fp32 (numpy ``float32``) for the INT8 encoder, explicit
boolean visibility masks, no tiling, no fusion, no reordering beyond what the
definitions state.  Each function names the passage of the source pages it
follows; the pages are

* [K25-arch]  "Kimi K2.5 model architecture deep-dive: industrial optimisation
  for ultra-long context" (framerc.cn),
* [MiMo-inf]  the IT之家 article on the Xiaomi MiMo-V2.5 inference system
  (hnjmgj.com),
* [S35-K25]   "2026 LLM architecture overview (III): Step 3.5 Flash & Kimi
  K2.5" (codearts.csdn.net).

Pins (tests marked ``not gpu``) tie every function to something other than
itself: brute force, library routines, closed forms and the pages' numbers.
No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    default_scale,
    visible_prefill,
    attend_masked,
    swa_prefill,
    swa_decode,
    attn_decode_int8kv,
    blocksparse_visible,
    blocksparse_attend,
)
from .ring import ring_slot, ring_fill, ring_append, ring_positions  # noqa: F401
from .prefix import window_safe_len  # noqa: F401
from .chunk import swa_prefill_chunk  # noqa: F401
from .sparse_decode import int8_block_means, sparse_select, attn_decode_int8kv_sparse  # noqa: F401
from .quant import kv_quant_int8_b32, dequant_int8_b32  # noqa: F401
from .select import block_sums, block_scores, block_select  # noqa: F401
from .closed_forms import (  # noqa: F401
    visible_pairs_prefill,
    attention_flops,
    hybrid_kv_ratio,
    hybrid_prefill_pair_ratio,
)
