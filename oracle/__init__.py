"""fp64 CPU oracle for fused softmax cross-entropy, row-wise softmax and
cross-entropy over vocabulary shards.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path.
"""
from .ce_oracle import (  # noqa: F401
    ce,
    ce_rows,
    ce_rows_ignore,
    reduce_loss,
    rne_bf16_bits,
    rne_f16_bits,
    widen_bf16,
    widen_f16,
)
from .softmax_oracle import (  # noqa: F401
    combine_partials,
    shard_partials,
    softmax_bwd_rows,
    softmax_rows,
)
