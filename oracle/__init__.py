"""CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
link this package. The only permitted users are ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``.

The oracle is the plain definition of what the hot path computes, written
out in float64 numpy (pure-Python loops only for the brute-force check on
tiny inputs). It shares no code with the HIP library: no kernels, headers,
helpers or constants. The two meet only through the seeded inputs that
``workloads`` produces and that callers pass to both sides.

Modules
  attention  paged decode, decode over an unpaged (contiguous) cache,
             chunked-prefill and latent (MLA-style) decode attention, KV
             append (write) and block copy
  pages      page / block-table arithmetic of the admission ledger

Every function names the passage of the pages it follows. No function here
is "parity unpinned": each is pinned in ``tests/test_oracle_*.py`` and
``tests/test_pages.py`` against page facts, brute force, a library routine,
closed forms or invariants.
"""

from .attention import (  # noqa: F401
    BLOCK_SIZE,
    as_f64,
    round_to_bf16_bits,
    gather_sequence,
    decode_contiguous,
    paged_decode,
    contiguous_cache_decode,
    paged_prefill,
    latent_decode,
    brute_force_decode,
    write_kv,
    copy_blocks,
)
from . import pages  # noqa: F401
