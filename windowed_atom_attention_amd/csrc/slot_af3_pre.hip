// slot_af3_pre.hip -- AF3 slot-attention kernels that read the pair bias
// precomputed by the projection kernel (fp32 and bf16 storage).
#include "slot_kernel.hpp"

namespace waa {

const void *pick_slot_af3_pre(int dtype, int spl, int D) {
    return dtype == 0 ? pick_slot_sd<float, STYLE_AF3, 0, 32>(spl, D)
                      : pick_slot_sd<bf16_t, STYLE_AF3, 0, 32>(spl, D);
}

} // namespace waa
