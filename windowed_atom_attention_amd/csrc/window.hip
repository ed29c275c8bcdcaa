// window.hip -- atom_attn_window_table: the windowed slot table built on the
// device, so that a caller whose key lists are local windows does not build
// and upload [B,A,K] ids from the host.
//
// Block q0 = block*floor(a/block) of queries sees the K consecutive key ids
// q0 - (K-block)/2 + k, k = 0..K-1, the window centred on its block (the
// layout the windowed workloads use). Ids outside [0, A), and with
// radius >= 0 ids farther than radius from the query, are written as -1:
// the block call treats both as missing slots ("windowed_atom_attention",
// Required behavior: the slot-permission and radius bullets), so folding
// the radius in here changes no result. Ids are int64 (the block's input
// type) or int32.
//
// One thread writes 16 bytes (two int64 or four int32 ids) of a row when
// the row length allows it, so every store is a full 16-byte vector of a
// coalesced stream; rows of other lengths are written one id per thread.
#include "../../include/atom_attn.h"
#include "kernels.hpp"

namespace waa {

template <typename I, int VEC>
__global__ __launch_bounds__(256) void k_window(I *out, uint32_t nvec, uint32_t per_row, int A,
                                                int K, int block, int64_t radius) {
    // 32-bit index arithmetic: B*A*K < 2^31 ids (checked by the entry point)
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    if (t >= nvec)
        return;
    const uint32_t row = t / per_row;
    const int k0 = (int)(t - row * per_row) * VEC;
    const int a = (int)(row % (uint32_t)A);
    // floor((K - block) / 2), also when K < block
    const int off = K - block;
    const int half = off >= 0 ? off / 2 : -((-off + 1) / 2);
    const int start = (a / block) * block - half;
    I v[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const int j = start + k0 + e;
        const int dist = j > a ? j - a : a - j;
        const bool ok = j >= 0 && j < A && (radius < 0 || dist <= radius);
        v[e] = ok ? (I)j : (I)-1;
    }
    I *dst = out + (size_t)row * K + k0;
    if constexpr (VEC * sizeof(I) == 16) {
        uint4 w;
        __builtin_memcpy(&w, v, 16);
        *reinterpret_cast<uint4 *>(dst) = w;
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            dst[e] = v[e];
    }
}

template <typename I, int VEC>
hipError_t launch_window(void *out, int64_t nrows, int A, int K, int block, int64_t radius,
                         hipStream_t s) {
    const int64_t threads = nrows * (K / VEC);
    const int64_t grid = (threads + 255) / 256;
    ProfSpan sp = prof_begin(KN_WINDOW, s);
    hipLaunchKernelGGL((k_window<I, VEC>), dim3((unsigned)grid), dim3(256), 0, s, (I *)out,
                       (uint32_t)threads, (uint32_t)(K / VEC), A, K, block, radius);
    prof_end(sp, s);
    return hipGetLastError();
}

} // namespace waa

extern "C" int atom_attn_window_table(int64_t B, int64_t A, int64_t K, int64_t block,
                                      int64_t radius, int index_bytes, void *key_index,
                                      void *stream) {
    using namespace waa;
    if (B < 1 || A < 1 || K < 1 || block < 1 || radius < -1 || !key_index ||
        (index_bytes != 4 && index_bytes != 8))
        return ATOM_ATTN_EINVAL;
    // ids fit the index type, and the grid fits one launch dimension
    if (A > ((int64_t)1 << 29) || K > ((int64_t)1 << 20) || block > ((int64_t)1 << 29) ||
        B * A * K >= ((int64_t)1 << 31))
        return ATOM_ATTN_EUNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const int64_t nrows = B * A;
    const bool vec = ((uintptr_t)key_index & 15) == 0 && (K * index_bytes) % 16 == 0;
    hipError_t e;
    if (index_bytes == 8)
        e = vec ? launch_window<int64_t, 2>(key_index, nrows, (int)A, (int)K, (int)block, radius, s)
                : launch_window<int64_t, 1>(key_index, nrows, (int)A, (int)K, (int)block, radius, s);
    else
        e = vec ? launch_window<int32_t, 4>(key_index, nrows, (int)A, (int)K, (int)block, radius, s)
                : launch_window<int32_t, 1>(key_index, nrows, (int)A, (int)K, (int)block, radius, s);
    return e == hipSuccess ? ATOM_ATTN_OK : ATOM_ATTN_ELAUNCH;
}
