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
// there, 16 lanes per token, which also sum the squares for the key/query
// norms); outputs of a block are gathered in LDS and written back as
// contiguous rows.
//
// Per token t one pass over the state forms both S_{t-1} k_t and the previous
// token's output S_{t-1} q_{t-1} (two independent dot products per lane, summed
// over the 4 lanes of a row by DPP), and a second pass applies the rank-1
// update with the key held in registers.  The decay is kept as a running
// scalar: S = c R, so that a token costs one FMA per state element instead of
// a multiply and an FMA; c is folded back into R at the end of each block, or
// at once if it falls below 2^-30 (bounding 1/c).
#include "gdn_launch.h"
#include "gdn_numeric.h"

namespace gdn {
namespace {

constexpr int kLanesPerRow = 4;
constexpr int kTB = 16;   // tokens staged per block
constexpr int kPPT = 16;  // staging lanes per token

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
// Sum over the 4 lanes of a quad (every lane receives it).
__device__ __forceinline__ float quad_sum(float x) {
    x += dpp_f<0xB1>(x);  // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);  // quad_perm [2,3,0,1]
    return x;
}
// Sum over 16 aligned lanes (every lane receives it).
__device__ __forceinline__ float row16_sum(float x) {
    x = quad_sum(x);
    x += dpp_f<0x141>(x);  // row_half_mirror
    x += dpp_f<0x140>(x);  // row_mirror
    return x;
}

// Maximum over 16 aligned lanes of non-negative values (every lane receives it).
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x141>(x));
    x = fmaxf(x, dpp_f<0x140>(x));
    return x;
}

template <int DK, int DV, int DVB, typename T>
__global__ __launch_bounds__(kLanesPerRow * DVB, 4)  // four waves per SIMD
void recurrent_kernel(const LaunchDesc P)
{
    constexpr int NT = kLanesPerRow * DVB;
    constexpr int E = DK / kLanesPerRow;       // state elements per lane
    constexpr int E4 = E / 4;                  // float4 groups per lane
    constexpr int NBLK = DV / DVB;
    constexpr int CPT = DK / kPPT;             // staged columns per lane and token
    // key/query row stride = 16 (mod 64) words, so that the four tokens staged
    // by one wave land on different banks
    constexpr int SK = DK + ((16 - DK) & 63);
    static_assert(E % 4 == 0 && CPT >= 1, "d_k must be a multiple of 16");
    static_assert((kTB * kPPT) % NT == 0, "staging passes cover whole waves");
    static_assert((kTB * DVB) % NT == 0, "value staging covers whole waves");

    __shared__ __attribute__((aligned(16))) float sk[kTB][SK];
    __shared__ __attribute__((aligned(16))) float sq[kTB][SK];
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
    const bool norm_k = (P.flags & kNormK) != 0, norm_q = (P.flags & kNormQ) != 0;
    const int H = P.H;

    // Lane `sub` owns key columns (g*4 + sub)*4 .. +3 for g in [0, E4): four
    // neighbouring lanes read 64 contiguous bytes per step (no bank conflicts).
    // The state is S = c R.
    float4 R[E4];
    float c = 1.f;
    if (wf & kWorkIdentity) {
#pragma unroll
        for (int g = 0; g < E4; ++g) {
            const int c0 = (g * kLanesPerRow + sub) * 4;
            R[g] = make_float4(c0 == grow ? 1.f : 0.f, c0 + 1 == grow ? 1.f : 0.f, c0 + 2 == grow ? 1.f : 0.f,
                               c0 + 3 == grow ? 1.f : 0.f);
        }
    } else if (P.init_off[r] >= 0) {
        const float *src = P.init_base + P.init_off[r] + (int64_t)h * DV * DK + (int64_t)grow * DK;
#pragma unroll
        for (int g = 0; g < E4; ++g)
            R[g] = *reinterpret_cast<const float4 *>(src + (g * kLanesPerRow + sub) * 4);
    } else {
#pragma unroll
        for (int g = 0; g < E4; ++g) R[g] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const int len = P.len[r];
    const int64_t row0 = P.row0[r];
    int ne = P.emit_begin[r];
    const int ne_end = P.emit_begin[r + 1];
    int next_emit = ne < ne_end ? P.emit_after[ne] : -1;  // span position of the next emission
    const T *qg = static_cast<const T *>(P.q);
    const T *kg = static_cast<const T *>(P.k);
    const T *vg = static_cast<const T *>(P.v);
    const T *ag = static_cast<const T *>(P.alpha);
    const T *bg = static_cast<const T *>(P.beta);
    T *og = static_cast<T *>(P.o);

    // R . x over a lane's columns, two accumulators
    auto dot = [&](const float4 (&x)[E4]) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int g = 0; g < E4; ++g) {
            d0 = fmaf(R[g].x, x[g].x, d0);
            d1 = fmaf(R[g].y, x[g].y, d1);
            d0 = fmaf(R[g].z, x[g].z, d0);
            d1 = fmaf(R[g].w, x[g].w, d1);
        }
        return d0 + d1;
    };
    // R . (row of LDS), the row read one group at a time
    auto dot_lds = [&](const float *row) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int g = 0; g < E4; ++g) {
            const float4 x = *reinterpret_cast<const float4 *>(row + (g * kLanesPerRow + sub) * 4);
            d0 = fmaf(R[g].x, x.x, d0);
            d1 = fmaf(R[g].y, x.y, d1);
            d0 = fmaf(R[g].z, x.z, d0);
            d1 = fmaf(R[g].w, x.w, d1);
        }
        return d0 + d1;
    };
    auto load_row = [&](const float *row, float4 (&x)[E4]) {
#pragma unroll
        for (int g = 0; g < E4; ++g) x[g] = *reinterpret_cast<const float4 *>(row + (g * kLanesPerRow + sub) * 4);
    };
    auto store_scaled = [&](float *dst, float sc) {
#pragma unroll
        for (int g = 0; g < E4; ++g) {
            const float4 x = R[g];
            *reinterpret_cast<float4 *>(dst + (g * kLanesPerRow + sub) * 4) =
                make_float4(x.x * sc, x.y * sc, x.z * sc, x.w * sc);
        }
    };

    for (int t0 = 0; t0 < len; t0 += kTB) {
        const int nt = min(kTB, len - t0);
        __syncthreads();
        // Staging.  Every global load of the block is issued before the first
        // use.  Lanes of tokens past the block read its last row (always in the
        // span) and store zeros.  Keys and queries: lanes 16 t .. 16 t + 15 of
        // a pass take token t (columns part, part + 16, ...) and sum its squares.
        constexpr int KPASS = kTB * kPPT / NT >= 1 ? kTB * kPPT / NT : 1;
        constexpr int VPL = kTB * DVB / NT;  // value loads per lane (= kTB / 4)
        float xk[KPASS][CPT], xq[KPASS][CPT], vx[VPL];
        float xa = 0.f, xb = 0.f;
#pragma unroll
        for (int ps = 0; ps < KPASS; ++ps) {
            const int idx = tid + NT * ps, t = min(idx / kPPT, nt - 1), part = idx % kPPT;
            const int64_t base = ((row0 + t0 + t) * H + h) * DK + part;
#pragma unroll
            for (int i = 0; i < CPT; ++i) xk[ps][i] = to_f32(kg[base + kPPT * i]);
        }
        if (want_o) {
#pragma unroll
            for (int ps = 0; ps < KPASS; ++ps) {
                const int idx = tid + NT * ps, t = min(idx / kPPT, nt - 1), part = idx % kPPT;
                const int64_t base = ((row0 + t0 + t) * H + h) * DK + part;
#pragma unroll
                for (int i = 0; i < CPT; ++i) xq[ps][i] = to_f32(qg[base + kPPT * i]);
            }
        }
        if (!zero_v) {
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int idx = tid + NT * i, t = min(idx / DVB, nt - 1), cc = idx % DVB;
                vx[i] = to_f32(vg[((row0 + t0 + t) * H + h) * DV + blk * DVB + cc]);
            }
        }
        if (tid < nt) {
            const int64_t ab = (row0 + t0 + tid) * H + h;
            xa = to_f32(ag[ab]);
            xb = to_f32(bg[ab]);
        }
        // A row that is normalised is stored scaled by the power of two that
        // brings its largest element into [1/2, 1) (exact), so that its sum of
        // squares lies in [1/4, d] and neither overflows (||x|| above ~1.8e19
        // in float32) nor underflows; the stored scale is 1/||scaled row||, and
        // a zero row keeps scale 0.
        auto stage_row = [&](const float (&x)[CPT], bool live, bool norm, float *dst, float *scale_out) {
            float y[CPT];
            int E = 0;
            if (norm) {
                float mx = 0.f;
#pragma unroll
                for (int i = 0; i < CPT; ++i) mx = fmaxf(mx, live ? fabsf(x[i]) : 0.f);
                E = __builtin_amdgcn_frexp_expf(row16_max(mx));
            }
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                y[i] = live ? __builtin_amdgcn_ldexpf(x[i], -E) : 0.f;
                dst[kPPT * i] = y[i];
                ss = fmaf(y[i], y[i], ss);
            }
            ss = row16_sum(ss);
            *scale_out = norm ? inv_norm(ss) : 1.f;
        };
#pragma unroll
        for (int ps = 0; ps < KPASS; ++ps) {
            const int idx = tid + NT * ps, t = idx / kPPT, part = idx % kPPT;
            const bool live = t < nt;
            float kn, qn = 1.f;
            stage_row(xk[ps], live, norm_k, &sk[t][part], &kn);
            if (want_o) stage_row(xq[ps], live, norm_q, &sq[t][part], &qn);
            if (part == 0 && live) {
                skn[t] = kn;
                sqn[t] = qn;
            }
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int idx = tid + NT * i, t = idx / DVB;
            sv[t][idx % DVB] = (t < nt && !zero_v) ? vx[i] : 0.f;
        }
        if (tid < nt) {
            sa[tid] = xa;
            sb[tid] = xb;
        }
        __syncthreads();

#pragma unroll 2
        for (int t = 0; t < nt; ++t) {
            float4 kv[E4];
            load_row(sk[t], kv);
            float u;
            if (want_o && t > 0) {
                // the output of token t - 1 comes from the same state S_{t-1}
                u = dot(kv);
                const float p = quad_sum(dot_lds(sq[t - 1]));
                if (sub == 0) so[t - 1][lrow] = p * c * sqn[t - 1];
            } else {
                u = dot(kv);
            }
            u = quad_sum(u);
            const float a = sa[t], kn = skn[t];
            const float ut = c * kn * u;  // S_{t-1} k^_t
            float cn = c * a;
            if (cn < 0x1p-30f) {
                // apply the decay now, so that 1/c stays bounded
#pragma unroll
                for (int g = 0; g < E4; ++g) {
                    R[g].x *= cn;
                    R[g].y *= cn;
                    R[g].z *= cn;
                    R[g].w *= cn;
                }
                cn = 1.f;
            }
            // S_t = a S_{t-1} + beta (v - a S_{t-1} k^) k^^T = cn (R + wr k_t^T) with the raw key
            // (1/cn to within an ulp: a relative error of 1e-7 in one token's update)
            const float wr = sb[t] * (sv[t][lrow] - a * ut) * kn * __builtin_amdgcn_rcpf(cn);
#pragma unroll
            for (int g = 0; g < E4; ++g) {
                R[g].x = fmaf(wr, kv[g].x, R[g].x);
                R[g].y = fmaf(wr, kv[g].y, R[g].y);
                R[g].z = fmaf(wr, kv[g].z, R[g].z);
                R[g].w = fmaf(wr, kv[g].w, R[g].w);
            }
            c = cn;
            if (next_emit == t0 + t + 1) {
                store_scaled(P.emit_base + ((((int64_t)b * P.M + P.emit_slot[ne]) * H + h) * DV + grow) * DK, c);
                ++ne;
                next_emit = ne < ne_end ? P.emit_after[ne] : -1;
            }
        }
        if (want_o) {
            // output of the block's last token
            const float p = quad_sum(dot_lds(sq[nt - 1]));
            if (sub == 0) so[nt - 1][lrow] = p * c * sqn[nt - 1];
        }
        // fold the decay back into the state once per block
#pragma unroll
        for (int g = 0; g < E4; ++g) {
            R[g].x *= c;
            R[g].y *= c;
            R[g].z *= c;
            R[g].w *= c;
        }
        c = 1.f;
        if (want_o) {
            __syncthreads();
            for (int idx = tid; idx < nt * DVB; idx += NT) {
                const int t = idx / DVB, cc = idx % DVB;
                og[((row0 + t0 + t) * H + h) * DV + blk * DVB + cc] = from_f32<T>(so[t][cc]);
            }
        }
    }

    if (P.state_dst[r]) store_scaled(P.state_dst[r] + (int64_t)h * DV * DK + (int64_t)grow * DK, 1.f);
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
