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

// d = 128: each thread forms a 4 x 4 block of the result (rows 4 ty.., columns
// 4 tx..), so that two 16-byte LDS reads feed sixteen FMAs; the workgroup's 32
// rows of a are held transposed ([k][row]) and p passes in 32-row tiles.  The
// sums run over k in order, starting from c.
__global__ __launch_bounds__(256) void affine_combine128_kernel(const float *__restrict__ a,
                                                                const float *__restrict__ p,
                                                                const float *__restrict__ c,
                                                                float *__restrict__ out) {
    constexpr int D = 128, RB = 32, KT = 32;
    __shared__ __attribute__((aligned(16))) float saT[D][RB + 4];
    __shared__ __attribute__((aligned(16))) float sp[KT][D + 4];
    const int64_t pair = blockIdx.x;
    const int tid = threadIdx.x, tx = tid & 31, ty = tid >> 5;
    const int64_t off = pair * D * D + (int64_t)blockIdx.y * RB * D;
    const float4 *A4 = reinterpret_cast<const float4 *>(a + off);
    const float *Pm = p + pair * D * D;
    for (int i = tid; i < RB * D / 4; i += 256) {
        const float4 v = A4[i];
        const int row = (4 * i) / D, col = (4 * i) % D;
        saT[col][row] = v.x;
        saT[col + 1][row] = v.y;
        saT[col + 2][row] = v.z;
        saT[col + 3][row] = v.w;
    }
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 cv = *reinterpret_cast<const float4 *>(c + off + (4 * ty + i) * D + 4 * tx);
        acc[i][0] = cv.x;
        acc[i][1] = cv.y;
        acc[i][2] = cv.z;
        acc[i][3] = cv.w;
    }
    for (int k0 = 0; k0 < D; k0 += KT) {
        __syncthreads();  // the previous tile of p is consumed (and a is in place)
        const float4 *P4 = reinterpret_cast<const float4 *>(Pm + (int64_t)k0 * D);
        for (int i = tid; i < KT * D / 4; i += 256)
            *reinterpret_cast<float4 *>(&sp[(4 * i) / D][(4 * i) % D]) = P4[i];
        __syncthreads();
#pragma unroll 8
        for (int j = 0; j < KT; ++j) {
            const float4 av = *reinterpret_cast<const float4 *>(&saT[k0 + j][4 * ty]);
            const float4 pv = *reinterpret_cast<const float4 *>(&sp[j][4 * tx]);
            const float ar[4] = {av.x, av.y, av.z, av.w}, pr[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[r][q] = fmaf(ar[r], pr[q], acc[r][q]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4 *>(out + off + (4 * ty + i) * D + 4 * tx) =
            make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
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
        case 128: hipLaunchKernelGGL(affine_combine128_kernel, grid, dim3(256), 0, s, a, p, c, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gdn
