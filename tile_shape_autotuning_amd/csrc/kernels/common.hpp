// Device-side building blocks shared by the GEMM kernels (gfx950 / CDNA4).
//
// Everything here is written for 64-wide wavefronts and the CDNA4 matrix
// cores.  Lane layouts of the MFMA operands used below (verified on gfx950):
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) + e] and
//     B[8*(l/16) + e][l%16], e = 0..7; result D[4*(l/16) + r][l%16], r = 0..3.
//   v_mfma_f32_16x16x4_f32:   lane l holds A[l%16][l/16] and B[l/16][l%16];
//     result as above.
// Because the reduction index only has to agree between the two operands,
// any fixed assignment of k values to (lane group, element) is valid as long
// as A and B use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Kernel parameters (passed by value).  Matrices are row-major with natural
// leading dimensions: A [M][K], B [K][N], C [M][N]; bias [N] fp32 or null.
struct GemmParams {
    const void* A;
    const void* B;
    const float* bias;
    void* C;
    float* ws;            // split-K: fp32 partial sums, one [M x N] slab per split
    int64_t slab;         // floats from one split's slab to the next
    int M, N, K;
    int kps;              // K elements per split (multiple of the kernel's k unit)
    int split;            // number of K splits (grid blocks per output tile)
    int tiles_m, tiles_n;
    int out_bf16;         // 1: C is bf16, 0: C is fp32
    int act;              // 0 none, 1 ReLU, 2 GELU (erf form)
    int group_m;          // tile rows per scheduling group (>= 1)
    int slab_out;         // 1: sums go to the split slabs even with split == 1 (the padded path)
    int kb;               // rows of B in memory when fewer than K (rows kb .. K-1 read as zero); 0: K
    // stream-K kind: the first sk_dp tiles (in scheduling order) run one
    // workgroup each; the remaining sk_tail tiles' sk_ks K steps each are
    // spread evenly over sk_g further workgroups, whose pieces of a tile go to
    // slots of bm x bn floats (tile j, piece s at slot j * sk_smax + s) that a
    // second pass adds in piece order
    int sk_dp, sk_g, sk_tail, sk_ks, sk_smax;
};

// Buffer-resource word 3 for gfx9-family raw buffers (32-bit dwords, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;
// A voffset no buffer below reaches: loads there return zero (range check).
constexpr int kOOB = 0x7FFFFFF8;
// Largest num_records used, kept below kOOB so OOB lanes always fail the check.
constexpr int64_t kMaxRecords = 0x7FFFFF00;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes)
{
    int64_t n = bytes < 0 ? 0 : (bytes > kMaxRecords ? kMaxRecords : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, int voff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}

// The same load with the non-temporal cache policy (cache-policy operand 2 =
// nt on this chip family): for data the grid reads exactly once, which then
// does not displace lines that other workgroups re-read.
__device__ __forceinline__ u32x4_t load16_stream(__amdgpu_buffer_rsrc_t r, int voff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 2);
}

__device__ __forceinline__ unsigned short load2(__amdgpu_buffer_rsrc_t r, int voff)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
}

__device__ __forceinline__ unsigned load4(__amdgpu_buffer_rsrc_t r, int voff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 8x8 transpose of 16-bit elements held as 8 rows x 4 dwords (dword d of a row
// holds columns 2d, 2d+1).  Output column t (8 values, rows 0..7) goes to out[t].
__device__ __forceinline__ void transpose8x8_b16(const u32x4_t (&rows)[8], u32x4_t (&out)[8])
{
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const unsigned sel = (t & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            out[t][e] = __builtin_amdgcn_perm(rows[2 * e + 1][t >> 1], rows[2 * e][t >> 1], sel);
    }
}

// XOR swizzle of 16-byte chunks inside an LDS row of CPR chunks: row r, logical
// chunk c lives at physical chunk c ^ swz(r).  Chosen so that 16 consecutive
// rows at one logical chunk (an MFMA fragment read) hit distinct 16-byte bank
// groups within both a 128-byte and a 256-byte window.
template <int CPR>
__device__ __forceinline__ int swz(int r)
{
    static_assert(CPR == 4 || CPR == 8 || CPR == 16, "chunks per row");
    constexpr int s1 = (CPR == 4) ? 1 : 0;
    constexpr int s2 = s1 + ((CPR == 4) ? 2 : (CPR == 8) ? 3 : 4);
    return ((r >> s1) ^ (r >> s2)) & (CPR - 1);
}

// GELU in the erf form, 0.5 v (1 + erf(v / sqrt 2)), with the complementary
// error function of Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26: erfc(x) ~= (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) e^(-x^2),
// t = 1 / (1 + p x), x >= 0, absolute error <= 1.5e-7.  1 + erf(z) is taken as
// 2 - erfc(|z|) for z >= 0 and erfc(|z|) for z < 0, so the GELU error is at
// most 0.5 |v| 1.5e-7 plus fp32 rounding.  The bound is absolute only: far in
// the negative tail, where erfc itself falls below 1e-7, the approximation's
// relative error grows without a useful bound (both values there are far
// below anything a bf16 output or the tolerance resolves).  One reciprocal,
// one exponential and five FMAs: the
// library erff costs several times that, and the epilogue of a 256 x 256 tile
// evaluates it 65,536 times.
__device__ __forceinline__ float gelu_erf(float v)
{
    const float z = v * 0.70710678118654752f;
    const float az = fabsf(z);
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * az);
    const float poly =
        t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float q = poly * __expf(-az * az);   // erfc(|z|)
    return 0.5f * v * (z >= 0.0f ? 2.0f - q : q);
}

__device__ __forceinline__ float apply_act(float v, int act)
{
    if (act == 1)
        return v > 0.0f ? v : 0.0f;
    if (act == 2)
        return gelu_erf(v);
    return v;
}

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float v)
{
    return __builtin_bit_cast(unsigned short, static_cast<__bf16>(v));
}

// ---- split-K
// With split > 1 a block's sums skip bias, activation and conversion and go,
// as fp32, to its split's slab of the workspace (row-major, row stride N like
// C); a second kernel adds the slabs in split order and applies the rest.
// The padded path (shapes whose rows are not 16-byte multiples) does the same
// with any split: the kernel then runs on zero-padded copies of A and B and
// the second kernel writes the real C.
// Kernel boundaries order the two passes, so no flags or cache control are
// needed between them.
// Output (row, col) of the problem goes to dst[(row - row0) * ld + col - col0].
struct OutSpec {
    void* dst;
    const float* bias;
    int act;
    int bf16;
    int row0, col0;
    int64_t ld;
};

__device__ __forceinline__ OutSpec out_spec(const GemmParams& p, int split)
{
    if (p.split > 1 || p.slab_out)
        return OutSpec{p.ws + (int64_t)split * p.slab, nullptr, 0, 0, 0, 0, (int64_t)p.N};
    return OutSpec{p.C, p.bias, p.act, p.out_bf16, 0, 0, (int64_t)p.N};
}

// Wait until every vector memory access this wave issued has completed.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Block index -> (tile_m, tile_n, split).  The hardware hands consecutive
// workgroups to the 8 XCDs round robin; the first step renumbers blocks so
// that each XCD owns a contiguous range of logical ids (tiles that share A
// rows and B columns then share that XCD's L2).  Logical ids enumerate tiles
// split-major, and tiles in groups of group_m tile rows, column-major inside a
// group.
// Tile number (scheduling order) -> tile coordinates: groups of group_m tile
// rows, column-major inside a group.
__device__ __forceinline__ void tile_coords(int tile, int tiles_m, int tiles_n, int group_m, int& tm, int& tn)
{
    const int per_group = group_m * tiles_n;
    const int g = tile / per_group;
    const int first_m = g * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int in_g = tile - g * per_group;
    tm = first_m + in_g % gsize;
    tn = in_g / gsize;
}

__device__ __forceinline__ void map_block(int bid, int total, int tiles_m, int tiles_n, int group_m,
                                          int& tile, int& tm, int& tn, int& split)
{
    const int q = total >> 3, r = total & 7;
    const int x = bid & 7, i = bid >> 3;
    const int logical = x * q + (x < r ? x : r) + i;
    const int tiles = tiles_m * tiles_n;
    tile = logical % tiles;
    split = logical / tiles;
    tile_coords(tile, tiles_m, tiles_n, group_m, tm, tn);
}

// Stream-K partition of the sk_tail tiles' iterations (K steps) over sk_g
// workgroups: workgroup g takes iterations [g I / G, (g + 1) I / G),
// I = sk_tail * sk_ks.  The workgroup holding iteration x is the largest g
// with g I / G <= x, i.e. ((x + 1) G - 1) / I.
__device__ __forceinline__ int64_t sk_start(int64_t g, int64_t I, int64_t G) { return g * I / G; }
__device__ __forceinline__ int64_t sk_owner(int64_t x, int64_t I, int64_t G) { return ((x + 1) * G - 1) / I; }

}  // namespace tg
