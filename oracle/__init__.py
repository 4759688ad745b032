"""fp64 CPU oracle (test infrastructure only; see oracle.ragged)."""
from .ragged import (  # noqa: F401
    attend,
    attend_image_head,
    decode,
    kept_index,
    pack_attend_unpack,
    pack_rows,
    seqlens,
    unpack,
)
from .threshold_l2 import keep_rank, sq_norms, threshold_l2_mask  # noqa: F401,E402
from .projection import linear, out_projection, qkv_projection  # noqa: F401,E402
