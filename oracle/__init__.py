"""Float64 CPU oracle for the sparse MLA decode path, the cache store before it and the
indexer that produces its index lists.

TEST INFRASTRUCTURE: only tests/, the smoke check in __graft_entry__ and the
cpu_baseline leg of bench.py may import it.  The library never does; it shares no
code, constants or helpers with the HIP implementation.
"""

from .sparse_mla_oracle import (  # noqa: F401
    BF16_ENTRY_BYTES,
    FP8_ENTRY_BYTES,
    IDX_GLOBAL,
    IDX_LOGICAL,
    KV_BF16,
    KV_FP8_UE8M0,
    KV_FP8_TENSOR,
    QK_DIM,
    V_DIM,
    attend,
    bf16_bits_to_f64,
    chunk_bounds,
    decode_entries,
    e4m3fn_to_f64,
    merge_partials,
    page_bytes,
    sparse_mla_decode,
    sparse_mla_decode_partials,
    translate,
    ue8m0_to_f64,
)
from .cache_store_oracle import (  # noqa: F401,E402
    cache_store,
    e4m3fn_nearest,
    quantize_fp8_ue8m0,
    ue8m0_for_amax,
)
from .indexer_oracle import (  # noqa: F401,E402
    INDEX_DIM,
    KEY_BYTES,
    decode_keys,
    indexer_logits,
    indexer_topk,
    key_page_bytes,
    row_slots,
)
