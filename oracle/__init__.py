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
