// Prefill variant of the expert FFN (grouped bf16-MFMA GEMM); not built yet.
#include "common.hpp"
#include "plan.hpp"

namespace moe {

int prefill_tile_m() { return 128; }

int launch_prefill_ffn(int, const uint16_t*, const uint8_t*, const float*, const uint8_t*,
                       const float*, const SharedW&, const Plan&, int, int, int, int, int,
                       uint16_t*, float*, hipStream_t) {
    set_error("moe_fused_w8a16: the prefill variant is not available in this build");
    return MOE_EUNSUPPORTED;
}

}  // namespace moe
