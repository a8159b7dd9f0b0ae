"""CPU oracle for the paged sliding-window + clamped image-range attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) imports, links or calls this package; only the tests, the
package's ``smoke()`` check and the bench's CPU-baseline leg do.  It shares no
code with the GPU path: plain numpy, float64 for floating point, written from
the pages' definitions:

  * [SWA-MM]  vLLM PR #53147 summary (prhub.com.cn): restoring sliding-window
              tile pruning under a window-clamped multimodal-prefix mask.
  * [SLOT]    vllm-ascend Triton operator deep dive: ``_compute_slot_mapping_kernel``
              (0539edu.com): position -> physical KV slot through a block table.
  * [DCP]     MLA DCP decode two-stream overlap and V-up fusion study notes,
              vllm-ascend PR #16977 (huashanblog): history/current partials
              merged by log-sum-exp.

Every function is pinned by tests that do not re-derive it (printed values,
closed forms, textbook reductions, brute force); none is "parity unpinned".
"""
from .slot_mapping import slot_mapping_cp_ref, slot_mapping_ref  # noqa: F401
from .mask import allowed_ref, allowed_rows, row_interval_ref  # noqa: F401
from .tile_bounds import tile_bounds_ref  # noqa: F401
from .attention import attention_ref, attention_pruned_ref  # noqa: F401
from .lse_merge import lse_merge_ref  # noqa: F401
from .kv_cache import kv_cache_write_ref  # noqa: F401
from .vup import vup_projection_ref  # noqa: F401
