// draft_mfma.hip -- MFMA form of the draft strip kernel (bf16 factors).
#include "common.hpp"
#include "kernels.hpp"

namespace dspark {

bool mfma_supported(int r, dspark_dtype factor_dt) {
    (void)r;
    (void)factor_dt;
    return false;
}

hipError_t launch_draft_mfma_step(const DraftArgs&, const int32_t*, int, int, PartialBuf, int) {
    return hipErrorNotSupported;
}

}  // namespace dspark
