"""Plain fp64 CPU oracle for absorbed-MLA split-KV decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything here.  The
product path (the HIP library and its Python binding) never imports this
package and shares no code with it: the two meet only through the seeded input
generator, which holds none of the method's arithmetic.

Source pages: "Kimi K3 on AMD Instinct MI355X: vLLM serving ... on AgentX" (AMD
blog post, three translations).  Sections used:

* section 1 "Cache" (DCP8 paragraph): each decode-context-parallel shard returns
  a partial answer that carries its softmax normalisation, and the partial
  answers are merged with softmax weights;
* section 4 "MLA: AITER assembly long-context decode": query heads attend to the
  cached positions independently (padding heads changes no real head), and the
  history may be split into partitions whose results are combined, with the KV
  storage unchanged;
* section 1 "Cache" (payload estimate): one 576-value latent per position and layer,
  stored in FP8, appended to as the conversation grows (``cache.py``).

Every function says which of these it follows.  Where the pages are silent the
reading taken is stated in the docstring.  Parity is pinned in
``tests/test_oracle_pins.py`` against exact decimal brute force, closed forms,
library routines and the pages' own worked numbers.
"""

from .numerics import bf16_bits_to_f64, e4m3fn_codes_to_f64
from .cache import kv_append, quantize_e4m3fn, stored_row
from .attention import (
    D_LATENT,
    D_V,
    attention,
    decode,
    decode_paged,
    gather_latents,
    merge,
)

__all__ = [
    "D_LATENT",
    "D_V",
    "attention",
    "bf16_bits_to_f64",
    "decode",
    "decode_paged",
    "e4m3fn_codes_to_f64",
    "gather_latents",
    "kv_append",
    "merge",
    "quantize_e4m3fn",
    "stored_row",
]
