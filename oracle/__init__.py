"""CPU oracle for the top-k sparse MLA decode path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, fp64 statement of
what the GPU path computes.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path (the HIP
library and its Python binding) never does, and this package imports nothing
from the product path.

Sources (page titles as published):
  * "HiSparse" walkthrough (devpress.csdn.net) -- hot buffer, swap-in phases.
  * "5.1.1 · 从索引到 Kernel" (PaperTrace) -- index normalisation, online
    softmax, split-KV merge (equations (1)-(21)).
  * "PagedAttention 与 RadixAttention：上游机制与海光实现对照" -- decode
    attention definition, partition combine, shifted causal mask, paged
    grouped-query decode and prefix-extend attention over a token pool.
  * "[HiCache] TMA-staged host<->device KV transfer kernel (sm_90+)" -- the
    row copy between host and device pools.
  * "HiSparse" walkthrough and "5.1.1 · 从索引到 Kernel" §7.2 -- the 656-byte
    fp8_ds_mla latent rows and their dequantisation.
  * "5.1.1 · 从索引到 Kernel" §5.1 and §7.4 -- task tables of a ragged batch
    (plan / run) with stable row identity.

Pin status (what fixes each function other than itself) is listed in each
module header.  Every function here is pinned; none is "parity unpinned".
"""

from .normalize import candidate_set, normalize, block_view
from .hot_buffer import HotState, hot_lookup_swapin, hot_reset, backup_rows
from .attention import (
    bf16_bits_to_f64,
    attend_sparse,
    attend_partial,
    attend_dense_masked,
    attend_fsum,
    shifted_causal_mask,
    split_ranges,
)
from .merge import merge, merge_normalized
from .dense import decode_slots, extend_attention, extend_metadata, paged_gqa_decode
from .transfer import kv_transfer
from .fp8 import attend_sparse_fp8, dequant_rows, e4m3_to_f64, f32_to_bf16, reconstruct
from .plan import plan_tasks, run_tasks

__all__ = [
    "candidate_set", "normalize", "block_view",
    "HotState", "hot_lookup_swapin", "hot_reset", "backup_rows",
    "bf16_bits_to_f64", "attend_sparse", "attend_partial", "attend_dense_masked",
    "attend_fsum", "shifted_causal_mask", "split_ranges",
    "merge", "merge_normalized", "kv_transfer",
    "attend_sparse_fp8", "dequant_rows", "e4m3_to_f64", "f32_to_bf16", "reconstruct",
    "decode_slots", "extend_attention", "extend_metadata", "paged_gqa_decode",
    "plan_tasks", "run_tasks",
]
