// slot.hip -- host side of the slot-attention kernel (slot_kernel.hpp):
// shape support, LDS size, kernel choice and launch; and the transposed
// copy of v used by the standalone slot-attention entry point.
#include "slot_kernel.hpp"

namespace waa {

size_t slot_lds_bytes(const Dims &d, int dtype, int style) {
    (void)dtype;
    return slot_layout(d.H, d.V, style).total;
}

int slot_supported(const Dims &d, int dtype, int style) {
    const int esz = dtype ? 2 : 4;
    if ((d.D != 16 && d.D != 32 && d.D != 64 && d.D != 128) || d.K > 256)
        return 0;
    if (style == STYLE_AF3 && (d.V % 8 != 0 || d.V * esz > 64 || d.H > kHG))
        return 0;
    return slot_lds_bytes(d, dtype, style) <= kMaxLds;
}

hipError_t launch_slot(const SlotArgs &a0, int dtype, int style, hipStream_t s) {
    SlotArgs a = a0;
    // threads per query: 32 (the 512-thread form) for the AF3
    // precomputed-bias variant, which runs only on small grids, and for
    // ESMFold2 grids of at most two blocks per CU; 16 otherwise
    const int nblk = a.B * ((a.A + kQB - 1) / kQB);
    int tq;
    if (style == STYLE_AF3)
        tq = a.pbias != nullptr ? 32 : 16;
    else
        tq = nblk <= 2 * device_cus() ? 32 : 16;
    const int spl = slot_spl(a.K, tq);
    const Dims d{a.B, a.A, 1, a.K, 32, 32, a.H, a.D, a.V, 32, 32};
    const size_t lds = slot_lds_bytes(d, dtype, style);
    const void *fn;
    if (style == STYLE_AF3 && a.pbias != nullptr) {
        fn = pick_slot_af3_pre(dtype, spl, a.D);
    } else if (style == STYLE_AF3) {
        const int nv = a.V * (dtype ? 2 : 4) / 16;
        fn = dtype == 0 ? pick_slot_af3_f32(spl, a.D, nv) : pick_slot_af3_bf16(spl, a.D, nv);
    } else {
        fn = pick_slot_esm(dtype, spl, a.D, tq);
    }
    if (fn == nullptr)
        return hipErrorInvalidValue;
    allow_lds(fn, lds);
    const int grid = a.B * ((a.A + kQB - 1) / kQB);
    void *args[] = {(void *)&a};
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(kQB * tq), args, lds, s);
    if (e != hipSuccess)
        return e;
    return hipGetLastError();
}

// Transposed copy of v ([B][A][HD] -> [B][HD][vt_pitch(A)], zero padding
// included), for the standalone slot-attention entry point. Rows of
// unusable atoms are stored as zeros: the slot kernel multiplies whole key
// bands of V by probabilities that are zero off the allowed slots, so a
// NaN/Inf payload left in such a row would reach o as 0 * NaN.
template <typename T>
__global__ __launch_bounds__(256) void k_vt(const T *v, const uint8_t *usable, T *vt,
                                            int B, int A, int HD, int pitch, int *wide) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i == 0 && wide)
        wide[0] = 0;
    const int64_t per = (int64_t)A * HD;
    if (i >= per * B)
        return;
    const int64_t b = i / per;
    const int64_t r = i - b * per;
    const int aa = (int)(r / HD), c = (int)(r - (int64_t)aa * HD);
    const T x = v[i];
    vt[(b * HD + c) * pitch + aa] = usable[b * A + aa] ? x : (T)0;
    if (i < (int64_t)B * HD) // row i of the transposed copy: its zero padding
        for (int e = A; e < pitch; ++e)
            vt[i * pitch + e] = (T)0;
}

hipError_t launch_vt(const void *v, const uint8_t *usable, void *vt, int B, int A,
                     int HD, int dtype, int *wide, hipStream_t s) {
    const int64_t total = (int64_t)A * HD * B;
    const int64_t grid = (total + 255) / 256;
    if (dtype == 0)
        hipLaunchKernelGGL(k_vt<float>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const float *)v, usable, (float *)vt, B, A, HD, vt_pitch(A), wide);
    else
        hipLaunchKernelGGL(k_vt<bf16_t>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const bf16_t *)v, usable, (bf16_t *)vt, B, A, HD, vt_pitch(A), wide);
    return hipGetLastError();
}

} // namespace waa
