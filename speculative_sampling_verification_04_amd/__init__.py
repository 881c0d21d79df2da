"""specv: batched speculative-sampling verification on AMD MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI of libspecv.so
(include/specv.h); `binding` marshals torch tensors into that ABI.
"""
from .binding import (SpecvError, bonus_topk, geometric_fanout, load_library,  # noqa: F401
                      tree_verify, uniforms, verify, verify_cache, verify_ragged, verify_topk, version)
