"""CPU fp64 oracle for one-token decode attention with the Flash-Decoding
split/merge schedule.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The GPU library never calls it and shares no code, table or helper with it.

Sources (cited by page title and section):

* "M4.5 - Decode Attention Kernels, Mask Programs, and Backend Boundaries"
  (written M4.5 below): the decode definition (§0x01), the split-state algebra
  (§0x02A-§0x02H), split bounds and workspace ledgers (§0x03B-§0x03I), address
  translation (§0x04B-§0x04H), mask programs (§0x05A-§0x05D).
* "M5.4 - Long-Context KV Policies: Retention, Compression, and Budget
  Allocation" (M5.4): full-cache, sliding-window and sink+recent visible sets
  (§0x03-§0x05), dense and selected attention sharing one denominator
  (§0x02K).
* "M8.6 - Live-Data Quantization: Activations and KV Cache" (M8.6): the
  symmetric quantizer rule (§0x02A), scale placement inside attention
  (§0x03B, §0x03C), KIVI axes and residual (§0x06-§0x06C), the decoded
  reference attention (§0x0CA).

Pinning status: every public function is pinned by the CPU tests against
values the pages print, closed forms, invariants or brute force, except the
auto split heuristic, which lives in the GPU library and affects only speed.
"""
from .numerics import decode_bf16, decode_f16, decode_f32  # noqa: F401
from .visibility import visible_positions, visible_count, query_row_length  # noqa: F401
from .address import (  # noqa: F401
    nhd_offset, hnd_offset, paged_nhd_offset, paged_hnd_offset, paged_segments,
    ragged_nhd_offset, csr_page, ring_slot,
)
from .state import (  # noqa: F401
    State, EMPTY, merge_state, summarize_allowed, finalize, balanced_bounds,
    lse_merge, workspace_bytes_mlu, workspace_bytes_lse_o,
)
from .attend import attend, gather_rows, split_attend  # noqa: F401
from .quant import (  # noqa: F401
    quantize_symmetric_rows, write_int8_cache_oracle, quantized_count, kivi_empty_state,
    kivi_append, kivi_state_parts, kivi_state_from_parts,
)
from . import flashmask  # noqa: F401
