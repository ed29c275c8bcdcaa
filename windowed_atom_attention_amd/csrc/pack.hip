// pack.hip -- rearranges weight matrices into MFMA B-operand chunk order.
//
// A [kd x n] matrix (stored [in][out], row pitch ld) becomes, for each
// output block nb and each k-chunk kc, 64 lanes x 16 bytes, e < 16/sizeof(T):
//  * block layout (32x32 MFMA, 32 columns): lane (h = lane/32, c = lane%32)
//    holds W[kc*KC + h*HALF + e][nb*32 + c] (KC/HALF as in Mma32<T>);
//  * strip layout (16x16 MFMA, 16 columns): lane (g = lane/16, c = lane%16)
//    holds W[kc*KC + g*QUARTER + e][nb*16 + c] (KC/QUARTER as in Mma16<T>).
// A wave then fetches one chunk with a single fully coalesced 1 KB load.
// Layout: [nb][kc][lane].
#include "common.hpp"
#include "kernels.hpp"

namespace waa {

template <typename T>
__global__ __launch_bounds__(256) void k_pack(PackArgs a) {
    // the job of the workgroup's first unit (uniform: scalar reads of the
    // argument block), then of this thread's unit (a job spans at least 128
    // units, so at most a step or two further)
    const int64_t u0 = (int64_t)blockIdx.x * 256;
    int j = 0;
    while (j + 1 < a.njobs && u0 >= a.job[j + 1].dst)
        ++j;
    const int64_t u = u0 + threadIdx.x;
    if (u >= a.total)
        return;
    while (j + 1 < a.njobs && u >= a.job[j + 1].dst)
        ++j;
    const PackJob &jb = a.job[j];
    const int64_t local = u - jb.dst;
    const int lane = (int)(local & 63);
    const int64_t rest = local >> 6;
    const int KC = jb.strip ? Mma16<T>::KC : Mma32<T>::KC;
    const int nkc = jb.kd / KC;
    const int kc = (int)(rest % nkc);
    const int nb = (int)(rest / nkc);
    const T *src = reinterpret_cast<const T *>(jb.src);
    const int col = jb.strip ? nb * 16 + (lane & 15) : nb * 32 + (lane & 31);
    const int row0 = kc * KC + (jb.strip ? (lane >> 4) * Mma16<T>::QUARTER
                                         : (lane >> 5) * Mma32<T>::HALF);
    constexpr int E = 16 / sizeof(T);
    T vals[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        vals[e] = src[(int64_t)(row0 + e) * jb.ld + col];
    uint4 out;
    __builtin_memcpy(&out, vals, 16);
    a.out[u] = out;
}

hipError_t launch_pack(const PackArgs &a, int dtype, hipStream_t s) {
    if (a.total == 0)
        return hipSuccess;
    const int grid = (int)((a.total + 255) / 256);
    if (dtype == 0)
        hipLaunchKernelGGL(k_pack<float>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_pack<bf16_t>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace waa
