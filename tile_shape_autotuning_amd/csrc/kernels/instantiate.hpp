// Launch wrappers used by the generated instantiation units.
#pragma once

#include "gemm_skinny.hpp"
#include "gemm_tiled.hpp"
#include "gemm_tiled_dma.hpp"

namespace tg {

template <int BM, int BN, int BK, int WGM, int WGN, int ST, bool NTB, bool F32, int WK = 1>
hipError_t launch_tiled_dma(const GemmParams& p, int blocks, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_tiled_dma_kernel<BM, BN, BK, WGM, WGN, ST, NTB, F32, WK>), dim3(blocks),
                       dim3(64 * WGM * WGN * WK),
                       0, stream, p);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WGM, int WGN, int ST>
hipError_t launch_streamk(const GemmParams& p, int blocks, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_streamk_kernel<BM, BN, BK, WGM, WGN, ST>), dim3(blocks), dim3(64 * WGM * WGN), 0, stream,
                       p);
    return hipGetLastError();
}

template <bool BF, int BM, int BN, int BK, int WGM, int WGN, int ST>
hipError_t launch_tiled(const GemmParams& p, int blocks, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_tiled_kernel<BF, BM, BN, BK, WGM, WGN, ST>), dim3(blocks),
                       dim3(64 * WGM * WGN), 0, stream, p);
    return hipGetLastError();
}

template <int MT, int W, int U>
hipError_t launch_skinny(const GemmParams& p, int blocks, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_skinny_kernel<MT, W, U>), dim3(blocks), dim3(64 * W), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tg
