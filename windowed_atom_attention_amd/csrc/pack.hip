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
    // the block's first job: how many later jobs start at or before u0 (job
    // offsets ascend); independent scalar loads rather than a dependent chain
    int j = 0;
#pragma unroll
    for (int k = 1; k < kMaxPackJobs; ++k)
        j += (k < a.njobs && u0 >= a.job[k].dst) ? 1 : 0;
    const int64_t u = u0 + threadIdx.x;
    if (u >= a.total)
        return;
    // a job spans at least 128 units, so a block's lanes lie in job j, j+1
    // or j+2: uniform loads of the three, then a per-lane choice
    const int j1 = min(j + 1, kMaxPackJobs - 1), j2 = min(j + 2, kMaxPackJobs - 1);
    const bool in1 = j + 1 < a.njobs && u >= a.job[j1].dst;
    const bool in2 = j + 2 < a.njobs && u >= a.job[j2].dst;
    const PackJob &ja = a.job[j], &jb1 = a.job[j1], &jb2 = a.job[j2];
    const int64_t dst = in2 ? jb2.dst : (in1 ? jb1.dst : ja.dst);
    const int64_t ld = in2 ? jb2.ld : (in1 ? jb1.ld : ja.ld);
    const int kd = in2 ? jb2.kd : (in1 ? jb1.kd : ja.kd);
    const int strip = in2 ? jb2.strip : (in1 ? jb1.strip : ja.strip);
    const T *src = reinterpret_cast<const T *>(in2 ? jb2.src : (in1 ? jb1.src : ja.src));
    const int64_t local = u - dst;
    const int lane = (int)(local & 63);
    const int64_t rest = local >> 6;
    const int KC = strip ? Mma16<T>::KC : Mma32<T>::KC;
    const int nkc = kd / KC;
    const int kc = (int)(rest % nkc);
    const int nb = (int)(rest / nkc);
    const int col = strip ? nb * 16 + (lane & 15) : nb * 32 + (lane & 31);
    const int row0 = kc * KC + (strip ? (lane >> 4) * Mma16<T>::QUARTER
                                      : (lane >> 5) * Mma32<T>::HALF);
    constexpr int E = 16 / sizeof(T);
    T vals[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        vals[e] = src[(int64_t)(row0 + e) * ld + col];
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
