// Per-token float32 replay kernel for gfx950.
//
// Implements the state recurrence of "Tail-Replay: Escaping the Curse of
// Linear Attention in Prefix Caching for Hybrid LLMs" §2.3, eq. (1), with the
// d_v x d_k state right-multiplied by the key operator, in its rank-1 form
//     u = S k^,  S <- alpha S + beta (v - alpha u) k^^T,  o = S q^,
// token by token, entirely in float32.  It serves float32 inputs (where the
// chunked bf16 matrix-core kernel would not meet float32 accuracy) and every
// shape the chunked kernel does not cover.
//
// Work split: one workgroup per (request, head, block of DVB value rows),
// 4 lanes per row, each lane holding d_k/4 state elements in VGPRs.  Token
// inputs are staged through LDS in blocks of TB tokens (converted to float32
// there); the key/query norms are computed once per token in LDS; outputs of a
// block are gathered in LDS and written back as contiguous rows.
#include "gdn_launch.h"
#include "gdn_numeric.h"

namespace gdn {
namespace {

constexpr int kLanesPerRow = 4;
constexpr int kTB = 32;  // tokens staged per block

template <int DK, int DV, int DVB, typename T>
__global__ __launch_bounds__(kLanesPerRow * DVB)
void recurrent_kernel(const LaunchDesc P)
{
    constexpr int NT = kLanesPerRow * DVB;
    constexpr int E = DK / kLanesPerRow;       // state elements per lane
    constexpr int E4 = E / 4;                  // float4 groups per lane
    constexpr int NBLK = DV / DVB;
    static_assert(E % 4 == 0, "d_k must be a multiple of 16");

    __shared__ float sk[kTB][DK];
    __shared__ float sq[kTB][DK];
    __shared__ float sv[kTB][DVB];
    __shared__ float so[kTB][DVB];
    __shared__ float sa[kTB], sb[kTB], skn[kTB], sqn[kTB];

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int blk = L % NBLK;
    const int h = (L / NBLK) % P.H;
    const int r = L / (NBLK * P.H);
    const int b = P.req[r];
    const int tid = threadIdx.x;
    const int lrow = tid / kLanesPerRow;  // local value row
    const int sub = tid % kLanesPerRow;
    const int grow = blk * DVB + lrow;    // global value row
    const int wf = P.wflags[r];
    const bool want_o = P.o != nullptr && !(wf & kWorkNoOut);
    const bool zero_v = (wf & kWorkZeroV) != 0;
    const int H = P.H;

    // Lane `sub` owns key columns (g*4 + sub)*4 .. +3 for g in [0, E4): four
    // neighbouring lanes read 64 contiguous bytes per step (no bank conflicts).
    float4 S[E4];
    if (wf & kWorkIdentity) {
#pragma unroll
        for (int g = 0; g < E4; ++g) {
            const int c0 = (g * kLanesPerRow + sub) * 4;
            S[g] = make_float4(c0 == grow ? 1.f : 0.f, c0 + 1 == grow ? 1.f : 0.f, c0 + 2 == grow ? 1.f : 0.f,
                               c0 + 3 == grow ? 1.f : 0.f);
        }
    } else if (P.init_off[r] >= 0) {
        const float *src = P.init_base + P.init_off[r] + (int64_t)h * DV * DK + (int64_t)grow * DK;
#pragma unroll
        for (int g = 0; g < E4; ++g)
            S[g] = *reinterpret_cast<const float4 *>(src + (g * kLanesPerRow + sub) * 4);
    } else {
#pragma unroll
        for (int g = 0; g < E4; ++g) S[g] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const int len = P.len[r];
    const int64_t row0 = P.row0[r];
    int ne = P.emit_begin[r];
    const int ne_end = P.emit_begin[r + 1];
    const T *qg = static_cast<const T *>(P.q);
    const T *kg = static_cast<const T *>(P.k);
    const T *vg = static_cast<const T *>(P.v);
    const T *ag = static_cast<const T *>(P.alpha);
    const T *bg = static_cast<const T *>(P.beta);
    T *og = static_cast<T *>(P.o);

    for (int t0 = 0; t0 < len; t0 += kTB) {
        const int nt = min(kTB, len - t0);
        __syncthreads();
        for (int idx = tid; idx < nt * DK; idx += NT) {
            const int t = idx / DK, j = idx % DK;
            const int64_t base = ((row0 + t0 + t) * H + h) * DK + j;
            sk[t][j] = to_f32(kg[base]);
            if (want_o) sq[t][j] = to_f32(qg[base]);
        }
        for (int idx = tid; idx < nt * DVB; idx += NT) {
            const int t = idx / DVB, c = idx % DVB;
            sv[t][c] = zero_v ? 0.f : to_f32(vg[((row0 + t0 + t) * H + h) * DV + blk * DVB + c]);
        }
        if (tid < nt) {
            const int64_t ab = (row0 + t0 + tid) * H + h;
            sa[tid] = to_f32(ag[ab]);
            sb[tid] = to_f32(bg[ab]);
        }
        __syncthreads();
        if (tid < nt) {
            float kk = 0.f, qq = 0.f;
            for (int j = 0; j < DK; ++j) {
                kk += sk[tid][j] * sk[tid][j];
                if (want_o) qq += sq[tid][j] * sq[tid][j];
            }
            skn[tid] = (P.flags & kNormK) ? inv_norm(kk) : 1.f;
            sqn[tid] = (P.flags & kNormQ) ? inv_norm(qq) : 1.f;
        }
        __syncthreads();

        for (int t = 0; t < nt; ++t) {
            const float a = sa[t];
            const float kn = skn[t];
            float u = 0.f;
#pragma unroll
            for (int g = 0; g < E4; ++g) {
                const float4 kv = *reinterpret_cast<const float4 *>(&sk[t][(g * kLanesPerRow + sub) * 4]);
                u += S[g].x * kv.x + S[g].y * kv.y + S[g].z * kv.z + S[g].w * kv.w;
            }
            u += __shfl_xor(u, 1);
            u += __shfl_xor(u, 2);
            // w multiplies the raw key, so it carries the norm factor twice:
            // beta (v - alpha S k^) k^^T with k^ = kn * k.
            const float w = sb[t] * (sv[t][lrow] - a * (u * kn)) * kn;
#pragma unroll
            for (int g = 0; g < E4; ++g) {
                const float4 kv = *reinterpret_cast<const float4 *>(&sk[t][(g * kLanesPerRow + sub) * 4]);
                S[g].x = fmaf(w, kv.x, a * S[g].x);
                S[g].y = fmaf(w, kv.y, a * S[g].y);
                S[g].z = fmaf(w, kv.z, a * S[g].z);
                S[g].w = fmaf(w, kv.w, a * S[g].w);
            }
            if (want_o) {
                float p = 0.f;
#pragma unroll
                for (int g = 0; g < E4; ++g) {
                    const float4 qv = *reinterpret_cast<const float4 *>(&sq[t][(g * kLanesPerRow + sub) * 4]);
                    p += S[g].x * qv.x + S[g].y * qv.y + S[g].z * qv.z + S[g].w * qv.w;
                }
                p += __shfl_xor(p, 1);
                p += __shfl_xor(p, 2);
                if (sub == 0) so[t][lrow] = p * sqn[t];
            }
            if (ne < ne_end && P.emit_after[ne] == t0 + t + 1) {
                float *dst = P.emit_base +
                    ((((int64_t)b * P.M + P.emit_slot[ne]) * H + h) * DV + grow) * DK;
#pragma unroll
                for (int g = 0; g < E4; ++g)
                    *reinterpret_cast<float4 *>(dst + (g * kLanesPerRow + sub) * 4) = S[g];
                ++ne;
            }
        }
        if (want_o) {
            __syncthreads();
            for (int idx = tid; idx < nt * DVB; idx += NT) {
                const int t = idx / DVB, c = idx % DVB;
                og[((row0 + t0 + t) * H + h) * DV + blk * DVB + c] = from_f32<T>(so[t][c]);
            }
        }
    }

    if (P.state_dst[r]) {
        float *dst = P.state_dst[r] + (int64_t)h * DV * DK + (int64_t)grow * DK;
#pragma unroll
        for (int g = 0; g < E4; ++g)
            *reinterpret_cast<float4 *>(dst + (g * kLanesPerRow + sub) * 4) = S[g];
    }
}

template <int DK, int DV, typename T>
hipError_t launch_dims(const LaunchDesc &d, hipStream_t s)
{
    constexpr int DVB = DV < 64 ? DV : 64;
    int total_req_wg = d.nreq * d.H * (DV / DVB);
    if (total_req_wg == 0) return hipSuccess;
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, DVB, T>), dim3(total_req_wg),
                       dim3(kLanesPerRow * DVB), 0, s, d);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_type(const LaunchDesc &d, int dk, int dv, hipStream_t s)
{
#define GDN_CASE(DK_, DV_) \
    if (dk == DK_ && dv == DV_) return launch_dims<DK_, DV_, T>(d, s);
#define GDN_ROW(DK_) GDN_CASE(DK_, 16) GDN_CASE(DK_, 32) GDN_CASE(DK_, 64) GDN_CASE(DK_, 128)
    GDN_ROW(16) GDN_ROW(32) GDN_ROW(64) GDN_ROW(128)
#undef GDN_ROW
#undef GDN_CASE
    return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_recurrent(const LaunchDesc &d, int dk, int dv, Elem e, hipStream_t s)
{
    if (e == Elem::F32) return launch_type<float>(d, dk, dv, s);
    return launch_type<bf16_t>(d, dk, dv, s);
}

}  // namespace gdn
