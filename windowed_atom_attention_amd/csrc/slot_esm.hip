// slot_esm.hip -- ESMFold2 slot-attention kernels (no pair input), fp32 and
// bf16 storage.
#include "slot_kernel.hpp"

namespace waa {

const void *pick_slot_esm(int dtype, int spl, int D, int tq) {
    if (tq == 32)
        return dtype == 0 ? pick_slot_sd<float, STYLE_ESM, 1, 32>(spl, D)
                          : pick_slot_sd<bf16_t, STYLE_ESM, 1, 32>(spl, D);
    return dtype == 0 ? pick_slot_sd<float, STYLE_ESM, 1, 16>(spl, D)
                      : pick_slot_sd<bf16_t, STYLE_ESM, 1, 16>(spl, D);
}

} // namespace waa
