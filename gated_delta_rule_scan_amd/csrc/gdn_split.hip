// Combine step of the sequence-split prefill.
//
// "Tail-Replay: Escaping the Curse of Linear Attention in Prefix Caching for
// Hybrid LLMs" §2.3 splits the state after a span exactly: with the key
// operator on the right, S_end = S_start P + S^, where P = T_1 ... T_n is the
// product of the span's transitions and S^ the span's zero-start replay.  The
// split prefill computes P and S^ of a middle segment while the first segment
// runs, then forms the segment's end state here:
//     out = a p + c,   a, c, out: [d_v][d_k],  p: [d_k][d_k],  float32,
// one pair (request, head) per grid row, 32-row blocks of the result per
// workgroup.  The operands are tiled through LDS; this kernel moves
// 3 d_v d_k + d_k^2 floats per pair, a small fraction of the scans around it.
#include "gdn_launch.h"

namespace gdn {
namespace {

template <int D>
__global__ __launch_bounds__(256) void affine_combine_kernel(const float *__restrict__ a, const float *__restrict__ p,
                                                             const float *__restrict__ c, float *__restrict__ out) {
    constexpr int RB = D < 32 ? D : 32;  // result rows per workgroup
    constexpr int KT = D < 32 ? D : 32;  // rows of p per LDS tile
    constexpr int E = RB * D / 256;      // results per thread
    static_assert(E >= 1 && RB * D % 256 == 0, "256 threads cover the block");
    __shared__ float sa[RB][D + 1];
    __shared__ float sp[KT][D + 1];
    const int64_t pair = blockIdx.x;
    const int tid = threadIdx.x;
    const float *A = a + pair * D * D + (int64_t)blockIdx.y * RB * D;
    const float *C = c + pair * D * D + (int64_t)blockIdx.y * RB * D;
    float *O = out + pair * D * D + (int64_t)blockIdx.y * RB * D;
    const float *Pm = p + pair * D * D;
    for (int i = tid; i < RB * D; i += 256) sa[i / D][i % D] = A[i];
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = C[tid + 256 * e];
    for (int k0 = 0; k0 < D; k0 += KT) {
        __syncthreads();
        for (int i = tid; i < KT * D; i += 256) sp[i / D][i % D] = Pm[(int64_t)(k0 + i / D) * D + i % D];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int idx = tid + 256 * e, row = idx / D, col = idx % D;
            float s = 0.f;
#pragma unroll 8
            for (int j = 0; j < KT; ++j) s = fmaf(sa[row][k0 + j], sp[j][col], s);
            acc[e] += s;
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) O[tid + 256 * e] = acc[e];
}

}  // namespace

hipError_t launch_affine_combine(const float *a, const float *p, const float *c, float *out, int64_t npairs, int d,
                                 hipStream_t s) {
    if (npairs == 0) return hipSuccess;
    const int rb = d < 32 ? d : 32;
    const dim3 grid((unsigned)npairs, (unsigned)(d / rb));
    switch (d) {
        case 16: hipLaunchKernelGGL((affine_combine_kernel<16>), grid, dim3(256), 0, s, a, p, c, out); break;
        case 32: hipLaunchKernelGGL((affine_combine_kernel<32>), grid, dim3(256), 0, s, a, p, c, out); break;
        case 64: hipLaunchKernelGGL((affine_combine_kernel<64>), grid, dim3(256), 0, s, a, p, c, out); break;
        case 128: hipLaunchKernelGGL((affine_combine_kernel<128>), grid, dim3(256), 0, s, a, p, c, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gdn
