// Measurement helper, not part of the attention library's ABI: plain
// streaming-read kernels that give the practical HBM read ceiling the decode
// kernel is compared with (beside the 8 TB/s data-sheet figure).  Built into
// its own shared library (libkvc_probe.so) and used only by the benchmark.
//
//   kvcp_seq_read    every byte of a buffer once, 16 bytes per lane, grid-stride
//   kvcp_block_read  whole 4 KiB blocks in the order of a permutation, one wave
//                    per block group: the decode kernel's access pattern (one kv
//                    head of a 16-token block of 128 bf16 dims is 4 KiB)
//
// Either reads with plain loads or with the non-temporal hint (data used once,
// kept from displacing other lines in L2), which streams faster on gfx950.
//
//   kvcp_mfma_loop   back-to-back v_mfma_f32_32x32x16_bf16 on register operands
//                    (four independent accumulators per wave): the practical
//                    bf16 matrix rate the prefill kernel is compared with
//                    beside the 2.5 PFLOP/s data-sheet figure
//
// Both reduce what they read into one word per thread so that the loads are
// not removed; `out` needs grid * 256 uint32 words.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4* p) {
    if constexpr (NT)
        return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
    else
        return *p;
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void seq_read(const uint4* __restrict__ p, int64_t n16,
                                                uint32_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t acc = 0;
    for (int64_t base = (int64_t)blockIdx.x * 256 + threadIdx.x; base < n16; base += stride * U) {
        uint4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t i = base + k * stride;
            v[k] = i < n16 ? ld16<NT>(p + i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Wave w reads blocks perm[w*U .. w*U+U-1], then skips ahead by all waves.
template <int U, bool NT>
__global__ __launch_bounds__(256) void block_read(const uint4* __restrict__ p,
                                                  const int32_t* __restrict__ perm, int64_t nblk,
                                                  uint32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * 4;
    uint32_t acc = 0;
    for (int64_t b0 = w * U; b0 < nblk; b0 += nw * U) {
        uint4 v[U][4];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t b = b0 + k;
            const int64_t pb = b < nblk ? perm[b] : 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[k][j] = b < nblk ? ld16<NT>(p + pb * 256 + j * 64 + lane) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < U; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc ^= v[k][j].x ^ v[k][j].y ^ v[k][j].z ^ v[k][j].w;
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}


typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_loop(float* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)((float)((lane + i) & 7) * 0.125f);
        b[i] = (__bf16)((float)((lane * 3 + i) & 7) * 0.125f);
    }
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

template <bool NT>
hipError_t launch_seq(const uint4* p, int64_t n16, uint32_t* out, int grid, int unroll, hipStream_t st) {
    switch (unroll) {
        case 4: hipLaunchKernelGGL((seq_read<4, NT>), dim3(grid), dim3(256), 0, st, p, n16, out); break;
        case 8: hipLaunchKernelGGL((seq_read<8, NT>), dim3(grid), dim3(256), 0, st, p, n16, out); break;
        case 16: hipLaunchKernelGGL((seq_read<16, NT>), dim3(grid), dim3(256), 0, st, p, n16, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool NT>
hipError_t launch_block(const uint4* p, const int32_t* perm, int64_t nblk, uint32_t* out, int grid,
                        int unroll, hipStream_t st) {
    switch (unroll) {
        case 2: hipLaunchKernelGGL((block_read<2, NT>), dim3(grid), dim3(256), 0, st, p, perm, nblk, out); break;
        case 4: hipLaunchKernelGGL((block_read<4, NT>), dim3(grid), dim3(256), 0, st, p, perm, nblk, out); break;
        case 8: hipLaunchKernelGGL((block_read<8, NT>), dim3(grid), dim3(256), 0, st, p, perm, nblk, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// n16: buffer size in 16-byte units; unroll in {4, 8, 16}; nontemporal: 0 plain
// loads, 1 loads with the non-temporal hint.  Returns a hipError_t.
extern "C" int kvcp_seq_read(const void* p, int64_t n16, void* out, int grid, int unroll,
                             int nontemporal, void* stream) {
    if (!p || !out || n16 < 0 || grid < 1) return (int)hipErrorInvalidValue;
    const uint4* b = (const uint4*)p;
    hipStream_t st = (hipStream_t)stream;
    return (int)(nontemporal ? launch_seq<true>(b, n16, (uint32_t*)out, grid, unroll, st)
                             : launch_seq<false>(b, n16, (uint32_t*)out, grid, unroll, st));
}

// p holds nblk 4 KiB blocks; perm is a permutation of 0 .. nblk-1 (device,
// int32); unroll in {2, 4, 8}; nontemporal as above.  Returns a hipError_t.
extern "C" int kvcp_block_read(const void* p, const void* perm, int64_t nblk, void* out, int grid,
                               int unroll, int nontemporal, void* stream) {
    if (!p || !perm || !out || nblk < 0 || grid < 1) return (int)hipErrorInvalidValue;
    const uint4* b = (const uint4*)p;
    const int32_t* pm = (const int32_t*)perm;
    hipStream_t st = (hipStream_t)stream;
    return (int)(nontemporal ? launch_block<true>(b, pm, nblk, (uint32_t*)out, grid, unroll, st)
                             : launch_block<false>(b, pm, nblk, (uint32_t*)out, grid, unroll, st));
}

// grid workgroups of 4 waves, each wave iters x 4 matrix instructions of
// 32 x 32 x 16 (2 x 32 x 32 x 16 flops each); out needs grid * 256 floats.
// Returns a hipError_t.
extern "C" int kvcp_mfma_loop(void* out, int grid, int iters, void* stream) {
    if (!out || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_loop, dim3(grid), dim3(256), 0, (hipStream_t)stream, (float*)out, iters);
    return (int)hipGetLastError();
}
