"""MI355X-native MoE layer step with a GPU expert cache (HIP kernels for gfx950).

The compute lives in libexpert_cached_decode.so (see include/ec_api.h); this
package is its Python binding.
"""
from .binding import (EC_DT_BF16, EC_DT_F32, EC_DT_MXFP4, Context, ECError, PinnedBuffer,  # noqa: F401
                      bank_read, bank_write, cache_rebuild, expert_cache_step, last_step, layout, lib, make_shape,
                      moe_decode_block,
                      moe_decode_layer, moe_decode_layer_static, moe_gate_logits, moe_prefill_layer, moe_route,
                      workspace_size)
