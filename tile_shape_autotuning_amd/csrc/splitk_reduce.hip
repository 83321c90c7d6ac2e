// Second pass of split-K (page "Compilers and Kernel Languages", "A different
// tile for a different shape": split-K is one of the choices real kernels add
// for skinny problems).  The GEMM kernels leave one fp32 slab of raw sums per
// split in the workspace, row-major like C; this kernel adds the slabs in
// split order 0 .. S-1, then adds the bias, applies the activation, converts
// and stores C.  The activation is not linear, so it can only follow the
// complete sum.
//
// The pass is elementwise over the flattened M x N array: each thread owns
// four consecutive elements (one 16-byte load per slab), so every access is
// coalesced whatever the GEMM's tile shape was.  It reads S x M x N x 4 bytes
// and writes M x N elements: HBM-bound.  A thread issues the loads of all its
// slabs before the first add (with the split count a template argument the
// loads do not wait on one another; adding as each arrives would pay the
// memory latency S times), then adds them in split order, so the sum is the
// same as the one-at-a-time loop's.  Slabs are read once: non-temporal loads.
#include <hip/hip_runtime.h>

#include "kernels/common.hpp"
#include "runtime.hpp"

namespace tg {

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// S > 0: the split count, known at compile time; S == 0: `split` at run time.
template <int S>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* ws, int split, int64_t slab, int64_t mn, int n, const float* bias, void* C,
                     int out_bf16, int act, int vec_out)
{
    const int nsplit = S > 0 ? S : split;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
    for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < mn; i += stride) {
        const int cnt = mn - i < 4 ? (int)(mn - i) : 4;
        float v[4];
        if (cnt == 4) {
            f32x4_t s;
            if constexpr (S > 0) {
                f32x4_t part[S];
#pragma unroll
                for (int k = 0; k < S; ++k)
                    part[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(ws + k * slab + i));
                s = part[0];
#pragma unroll
                for (int k = 1; k < S; ++k)
                    s += part[k];
            } else {
                s = *reinterpret_cast<const f32x4_t*>(ws + i);
                for (int k = 1; k < nsplit; ++k)
                    s += *reinterpret_cast<const f32x4_t*>(ws + k * slab + i);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = s[e];
        } else {
            for (int e = 0; e < cnt; ++e) {
                float s = ws[i + e];
                for (int k = 1; k < nsplit; ++k)
                    s += ws[k * slab + i + e];
                v[e] = s;
            }
        }
        // the column of each element is only needed for the bias (a 64-bit
        // remainder on the path to the stores); without one the sums get
        // + 0.0f, as in the single-pass epilogue
        if (bias) {
            int col = (int)(i % n);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (e < cnt)
                    v[e] = v[e] + bias[col];
                col = col + 1 == n ? 0 : col + 1;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = v[e] + 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < cnt)
                v[e] = apply_act(v[e], act);
        if (out_bf16) {
            unsigned short* c = static_cast<unsigned short*>(C) + i;
            if (cnt == 4 && vec_out) {
                const u32x2_t w = {(unsigned)f32_to_bf16_rne(v[0]) | ((unsigned)f32_to_bf16_rne(v[1]) << 16),
                                   (unsigned)f32_to_bf16_rne(v[2]) | ((unsigned)f32_to_bf16_rne(v[3]) << 16)};
                *reinterpret_cast<u32x2_t*>(c) = w;
            } else {
                for (int e = 0; e < cnt; ++e)
                    c[e] = f32_to_bf16_rne(v[e]);
            }
        } else {
            float* c = static_cast<float*>(C) + i;
            if (cnt == 4 && vec_out) {
                *reinterpret_cast<f32x4_t*>(c) = f32x4_t{v[0], v[1], v[2], v[3]};
            } else {
                for (int e = 0; e < cnt; ++e)
                    c[e] = v[e];
            }
        }
    }
}

// Second pass of the stream-K kind: every tail tile whose K steps were split
// among two or more workgroups has its pieces, raw fp32 sums in bm x bn slots
// (tile j, piece s at slot j * smax + s), added in piece order -- which is K
// order -- then bias, activation and conversion, and the result stored in C.
// Tiles taken whole by one workgroup were finished by the GEMM kernel and are
// skipped.  One block row of the grid per tail tile; each thread owns four
// consecutive columns of a tile row (N is a multiple of 8 for this kind, so
// the four are inside or outside C together).
__global__ void __launch_bounds__(256)
streamk_fixup_kernel(const float* ws, int bm, int bn, int M, int N, int tiles_m, int tiles_n, int group_m, int dp,
                     int tail, int ks, int G, int smax, const float* bias, void* C, int out_bf16, int act)
{
    const int64_t j = blockIdx.y;
    const int64_t I = (int64_t)tail * ks;
    const int64_t first = sk_owner(j * ks, I, G);
    const int nseg = (int)(sk_owner((j + 1) * ks - 1, I, G) - first + 1);
    if (nseg < 2)
        return;
    int tm, tn;
    tile_coords(dp + (int)j, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t area = (int64_t)bm * bn;
    const float* base = ws + j * smax * area;
    for (int64_t e = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; e < area;
         e += (int64_t)gridDim.x * blockDim.x * 4) {
        const int r = (int)(e / bn), c = (int)(e % bn);
        const int row = tm * bm + r, col = tn * bn + c;
        if (row >= M || col >= N)
            continue;
        f32x4_t s = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(base + e));
        for (int k = 1; k < nseg; ++k)
            s += __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(base + k * area + e));
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[q] = apply_act(s[q] + (bias ? bias[col + q] : 0.0f), act);
        const int64_t idx = (int64_t)row * N + col;
        if (out_bf16) {
            const u32x2_t w = {(unsigned)f32_to_bf16_rne(v[0]) | ((unsigned)f32_to_bf16_rne(v[1]) << 16),
                               (unsigned)f32_to_bf16_rne(v[2]) | ((unsigned)f32_to_bf16_rne(v[3]) << 16)};
            *reinterpret_cast<u32x2_t*>(static_cast<unsigned short*>(C) + idx) = w;
        } else {
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(C) + idx) = f32x4_t{v[0], v[1], v[2], v[3]};
        }
    }
}

hipError_t streamk_fixup(const GemmParams& p, int bm, int bn, hipStream_t stream)
{
    const int per_tile = (int)(((int64_t)bm * bn / 4 + 255) / 256);
    hipLaunchKernelGGL(streamk_fixup_kernel, dim3(per_tile, p.sk_tail), dim3(256), 0, stream, p.ws, bm, bn, p.M, p.N,
                       p.tiles_m, p.tiles_n, p.group_m, p.sk_dp, p.sk_tail, p.sk_ks, p.sk_g, p.sk_smax, p.bias, p.C,
                       p.out_bf16, p.act);
    return hipGetLastError();
}

int64_t splitk_slab(int64_t M, int64_t N)
{
    // each slab starts 256-byte aligned, so 16-byte loads stay aligned
    return (M * N + 63) / 64 * 64;
}

hipError_t splitk_reduce(const float* ws, int split, int64_t M, int64_t N, const float* bias, void* C,
                         int out_bf16, int act, hipStream_t stream)
{
    const int64_t mn = M * N;
    if (mn <= 0)
        return hipSuccess;
    const int64_t want = (mn + 1023) / 1024;      // 256 threads x 4 elements per block
    const int blocks = (int)(want < 65536 ? want : 65536);
    // four outputs per store where C's alignment allows it (the element-load
    // kind accepts any C)
    const int vec_out = ((uintptr_t)C & (out_bf16 ? 7u : 15u)) == 0;
    const int64_t slab = splitk_slab(M, N);
#define TG_REDUCE(S)                                                                                          \
    hipLaunchKernelGGL(splitk_reduce_kernel<S>, dim3(blocks), dim3(256), 0, stream, ws, split, slab, mn, (int)N, \
                       bias, C, out_bf16, act, vec_out)
    switch (split) {
    case 2: TG_REDUCE(2); break;
    case 4: TG_REDUCE(4); break;
    case 8: TG_REDUCE(8); break;
    case 16: TG_REDUCE(16); break;
    default: TG_REDUCE(0); break;
    }
#undef TG_REDUCE
    return hipGetLastError();
}

}  // namespace tg
