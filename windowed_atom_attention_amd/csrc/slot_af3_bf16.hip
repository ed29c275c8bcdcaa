// slot_af3_bf16.hip -- AF3 slot-attention kernels, bf16 storage (pair rows
// of 8, 16, 24 or 32 channels: 1 to 4 16-byte vectors).
#include "slot_kernel.hpp"

namespace waa {

const void *pick_slot_af3_bf16(int spl, int D, int nv) {
    switch (nv) {
    case 1: return pick_slot_sd<bf16_t, STYLE_AF3, 1, 16>(spl, D);
    case 2: return pick_slot_sd<bf16_t, STYLE_AF3, 2, 16>(spl, D);
    case 3: return pick_slot_sd<bf16_t, STYLE_AF3, 3, 16>(spl, D);
    case 4: return pick_slot_sd<bf16_t, STYLE_AF3, 4, 16>(spl, D);
    default: return nullptr;
    }
}

} // namespace waa
