// The padded path of the tiled kind: GEMMs whose rows are not whole 16-byte
// chunks (K or N not a multiple of 8 bf16 / 4 fp32 elements).  The
// direct-to-LDS kernel moves 16-byte chunks of rows, so here it runs on
// zero-padded copies of the operands whose rows are ragged (or misaligned):
// A [M x K] -> A' [M x Kp], B [K x N] -> B' [Kp x Np], with Kp and Np
// rounded up to the chunk and the extra columns and rows zero, which adds
// nothing to any sum (a B read in place has the rows it lacks read as zero
// by the kernel's range check).  When N is ragged the kernel writes its fp32
// sums as split slabs [M x Np] (any split, 1 included), and the output pass
// below adds them in split order, adds the bias, applies the activation and
// writes the real C [M x N] element by element -- the same operations in the
// same order as the split-K second pass, so the results are those of the
// aligned kinds (page "Compilers and Kernel Languages", "A
// different tile for every shape": ragged shapes are where a fixed kernel
// loses; page "Tile Selection: Cost Models Against Measurement", "The
// structure of the search space": the tile grid covers the padded extents).
//
// Both passes move memory only: the copies read each operand once and write
// its padded form once (16-byte stores, the source read element by element
// since its rows start at any 2- or 4-byte boundary); the output pass reads
// each slab once with 16-byte loads and writes C.  Any pointer alignment is
// accepted on the caller's side.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels/common.hpp"
#include "runtime.hpp"

namespace tg {

namespace {

struct PadJob {
    const void* src;
    void* dst;
    int64_t rows;     // source rows (the rest of the destination rows are zero)
    int64_t rowsp;    // destination rows
    int64_t cols;     // source columns = source row stride
    int64_t colsp;    // destination columns = destination row stride (a multiple of 16 bytes)
};

// blockIdx.y picks the operand; the destination's 16-byte chunks, row after
// row, are spread over the threads (grid-stride), so short rows do not
// leave threads idle.  T: the element's bit pattern (2 or 4 bytes).
template <typename T>
__global__ void __launch_bounds__(256) pad_operands_kernel(PadJob a, PadJob b)
{
    const PadJob j = blockIdx.y == 0 ? a : b;
    constexpr int V = 16 / (int)sizeof(T);
    const T* src = static_cast<const T*>(j.src);
    T* dst = static_cast<T*>(j.dst);
    const int64_t chunks = j.colsp / V;       // per destination row
    const int64_t total = j.rowsp * chunks;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / chunks;
        const int64_t c0 = (i - r * chunks) * V;
        T v[V];
#pragma unroll
        for (int e = 0; e < V; ++e)
            v[e] = (r < j.rows && c0 + e < j.cols) ? src[r * j.cols + c0 + e] : T(0);
        u32x4_t w;
        __builtin_memcpy(&w, v, 16);
        *reinterpret_cast<u32x4_t*>(dst + i * V) = w;
    }
}

// S > 0: the split count at compile time; S == 0: `split` at run time.  Rows
// by blockIdx.y (grid-stride), four columns per thread: one 16-byte load per
// slab (ldp is a multiple of 4, so the four lie inside the padded row), then
// per column in range: sum in split order, + bias (or + 0), activation,
// conversion, store.
template <int S>
__global__ void __launch_bounds__(256)
padded_out_kernel(const float* ws, int split, int64_t slab, int64_t ldp, int64_t M, int64_t N, const float* bias,
                  void* C, int out_bf16, int act)
{
    const int nsplit = S > 0 ? S : split;
    for (int64_t r = blockIdx.y; r < M; r += gridDim.y) {
        for (int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; c0 < N; c0 += (int64_t)gridDim.x * 1024) {
            const float* src = ws + r * ldp + c0;
            f32x4_t s;
            if constexpr (S > 0) {
                f32x4_t part[S];
#pragma unroll
                for (int k = 0; k < S; ++k)
                    part[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src + k * slab));
                s = part[0];
#pragma unroll
                for (int k = 1; k < S; ++k)
                    s += part[k];
            } else {
                s = *reinterpret_cast<const f32x4_t*>(src);
                for (int k = 1; k < nsplit; ++k)
                    s += *reinterpret_cast<const f32x4_t*>(src + k * slab);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t c = c0 + e;
                if (c < N) {
                    const float v = apply_act(s[e] + (bias ? bias[c] : 0.0f), act);
                    if (out_bf16)
                        static_cast<unsigned short*>(C)[r * N + c] = f32_to_bf16_rne(v);
                    else
                        static_cast<float*>(C)[r * N + c] = v;
                }
            }
        }
    }
}

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

hipError_t pad_operands(const void* A, const void* B, void* Ap, void* Bp, int64_t M, int64_t N, int64_t K,
                        int64_t Np, int64_t Kp, int eb, bool copy_a, bool copy_b, hipStream_t stream)
{
    // an operand not copied gets a job of no rows
    const PadJob a{A, Ap, M, copy_a ? M : 0, K, Kp};
    const PadJob b{B, Bp, K, copy_b ? Kp : 0, N, Np};
    const int64_t v = 16 / eb;
    const int64_t most = std::max(a.rowsp * (Kp / v), b.rowsp * (Np / v));   // chunks of the larger copy
    const dim3 grid((unsigned)std::min<int64_t>(std::max<int64_t>(cdiv64(most, 256), 1), 4096), 2);
    if (eb == 2)
        hipLaunchKernelGGL(pad_operands_kernel<unsigned short>, grid, dim3(256), 0, stream, a, b);
    else
        hipLaunchKernelGGL(pad_operands_kernel<unsigned>, grid, dim3(256), 0, stream, a, b);
    return hipGetLastError();
}

hipError_t padded_output(const float* ws, int split, int64_t slab, int64_t ldp, int64_t M, int64_t N,
                         const float* bias, void* C, int out_bf16, int act, hipStream_t stream)
{
    if (M <= 0 || N <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)std::min<int64_t>(cdiv64(N, 1024), 64), (unsigned)std::min<int64_t>(M, 65535));
#define TG_PADDED_OUT(S)                                                                                          \
    hipLaunchKernelGGL(padded_out_kernel<S>, grid, dim3(256), 0, stream, ws, split, slab, ldp, M, N, bias, C, \
                       out_bf16, act)
    switch (split) {
    case 1: TG_PADDED_OUT(1); break;
    case 2: TG_PADDED_OUT(2); break;
    case 4: TG_PADDED_OUT(4); break;
    case 8: TG_PADDED_OUT(8); break;
    case 16: TG_PADDED_OUT(16); break;
    default: TG_PADDED_OUT(0); break;
    }
#undef TG_PADDED_OUT
    return hipGetLastError();
}

}  // namespace tg
