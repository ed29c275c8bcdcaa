// slot_af3_f32.hip -- AF3 slot-attention kernels, fp32 storage (pair rows
// of 8 or 16 channels: 2 or 4 16-byte vectors).
#include "slot_kernel.hpp"

namespace waa {

const void *pick_slot_af3_f32(int spl, int D, int nv) {
    switch (nv) {
    case 2: return pick_slot_sd<float, STYLE_AF3, 2, 16>(spl, D);
    case 4: return pick_slot_sd<float, STYLE_AF3, 4, 16>(spl, D);
    default: return nullptr;
    }
}

} // namespace waa
