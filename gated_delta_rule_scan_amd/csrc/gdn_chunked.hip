// Chunked matrix-core replay kernel for gfx950: bf16 inputs, float32 state,
// d_k = d_v = 128, normalised keys.
//
// The recurrence of "Tail-Replay: Escaping the Curse of Linear Attention in
// Prefix Caching for Hybrid LLMs" §2.3 eq. (1) (state d_v x d_k, key operator
// on the right) is advanced C = 64 tokens at a time.  Inside a chunk, with
// g_t = sum_{i<=t} ln alpha_i (chunk-local) and u_t = beta_t (v_t - alpha_t
// S_{t-1} k_t), unrolling eq. (1) gives
//     S_t = e^{g_t} S_0 + sum_{s<=t} e^{g_t - g_s} u_s k_s^T,
// and the u_t solve a unit lower-triangular system
//     (I + A) U = B,  A_ts = beta_t e^{g_t - g_s} (k_t . k_s)  (s < t),
//                     B_t  = beta_t (v_t - e^{g_t} S_0 k_t),
// so that, with T = (I + A)^{-1} (it depends on keys and gates only):
//     U   = T B
//     o_t = e^{g_t} S_0 q_t + sum_{s<=t} e^{g_t - g_s} (q_t . k_s) u_s
//     S_C = e^{g_C} S_0 + sum_s e^{g_C - g_s} u_s k_s^T.
// This is the compact-WY way of applying a product of rank-1 modifications of
// the identity (Golub & Van Loan, Matrix Computations, §5.1) to the chunk.
//
// Precision: the dense products run on fp16 MFMA (v_mfma_f32_32x32x16_f16 and
// v_mfma_f32_16x16x32_f16) with float32 accumulation.  Every fp16 operand is
// range-scaled by an exact power of two: keys/queries per token (k' = k/2^E
// with max|k'| < 1, exact for bf16 data), the state, B, U and T per wave or
// per chunk.  The triangular inverse T is formed in float32 on VALU.  The
// state itself never leaves float32.
//
// Work split: one workgroup of 4 waves per (request, head); wave w owns value
// rows [32w, 32w + 32).  The state is kept transposed, S^T (d_k x d_v), in
// MFMA accumulator layout; because the reduction index of an MFMA may be
// permuted freely (as long as both operands agree), each wave feeds its own
// accumulators back as B fragments of the next chunk's products, so the
// chunk-to-chunk chain of a wave never touches LDS for the state.
#include "gdn_launch.h"
#include "gdn_numeric.h"

namespace gdn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int C = 64;        // tokens per chunk
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int NW = 4;        // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int KST = DK + 4;  // row stride (halves) of kc / qc
constexpr int TST = C + 4;   // row stride (halves) of kct / vct / tc / pc
constexpr int AST = C + 4;   // row stride (floats) of aws

struct Smem {
    _Float16 kc[C * KST];     // k' = k / 2^E, token-major
    _Float16 qc[C * KST];     // q' = q / 2^E, token-major
    _Float16 kct[DK * TST];   // k', key-major
    uint16_t vct[DV * TST];   // v (bf16 bits), value-major
    _Float16 tc[C * TST];     // T scaled to fp16
    _Float16 pc[C * TST];     // P_ts = e^{g_t-g_s} kap_s (q'_t . k'_s), s <= t
    float aws[C * AST];       // A, then T, in float32
    float wws[32 * 33];       // scratch for the blocked inverse
    alignas(16) float beta[C];
    alignas(16) float g[C];               // ln alpha, then its chunk-local prefix sum
    alignas(16) float egk[C];             // e^{g_t} kap_t
    alignas(16) float eg[C];              // e^{g_t}
    alignas(16) float kap[C];             // 2^E_t / ||k_t||
    alignas(16) float kapq[C];            // 2^E_t / ||q_t|| (or 2^E_t)
    alignas(16) float wsc[C];             // e^{g_C - g_t} kap_t
    float red[NW];
    float egC;
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Power-of-two scale bringing max|x| into [2^14, 2^15): returns e with
// scale = 2^e, so that x * 2^e fits fp16 with full precision.
__device__ __forceinline__ int fp16_exp(float mx) {
    int E;
    frexpf(mx, &E);
    return 15 - E;
}

__device__ __forceinline__ float bf(uint16_t b) { return bf16_to_f32(b); }

__device__ __forceinline__ half4 ld4(const _Float16 *p) {
    return *reinterpret_cast<const half4 *>(p);
}

// A fragment of v_mfma_f32_32x32x16_f16 read from a row-major fp16 tile with
// the reduction index permuted as pi(k): lane i takes row `row`, columns
// c0 + 4*(i/32) + {0..3} and c0 + 8 + 4*(i/32) + {0..3}.
__device__ __forceinline__ half8 frag_perm(const _Float16 *base, int stride, int row, int c0, int lane) {
    const _Float16 *p = base + row * stride + c0 + 4 * (lane >> 5);
    half4 lo = ld4(p), hi = ld4(p + 8);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ half8 frag_contig(const _Float16 *p) {
    half4 lo = ld4(p), hi = ld4(p + 4);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Slots 8*half .. 8*half+7 of a 32x32 accumulator, scaled, as fp16.
__device__ __forceinline__ half8 to_frag(const floatx16 &acc, int half_, float scale) {
    half8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (_Float16)(acc[8 * half_ + j] * scale);
    return r;
}

__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// lower-triangular 16x16 tiles (mt, nt) of a 64 x 64 matrix, nt <= mt
__device__ __constant__ const int8_t kTileM[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__device__ __constant__ const int8_t kTileN[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};


// Store S (held as S^T tiles) to a d_v x d_k row-major float32 block.
__device__ __forceinline__ void store_state(float *dst_head, const floatx16 (&Sacc)[4], int w, int l32,
                                            int hi32) {
    float *dst = dst_head + (int64_t)(32 * w + l32) * DK;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<float4 *>(dst + 32 * a + 8 * q4 + 4 * hi32) =
                make_float4(Sacc[a][4 * q4], Sacc[a][4 * q4 + 1], Sacc[a][4 * q4 + 2], Sacc[a][4 * q4 + 3]);
}

// Chunk schedule: up to C tokens, cut at the next emission position.
__device__ __forceinline__ int chunk_len(const LaunchDesc &P, int len, int t0, int e, int e_end) {
    int lc = min(C, len - t0);
    if (e < e_end) lc = min(lc, P.emit_after[e] - t0);
    return lc;
}

// Raw loads of one chunk into registers.  Thread tid covers tokens
// 16 i + tid/16 (i = 0..3) and elements 8 (tid%16) .. +7 of q, k and v;
// threads 0..63 load alpha, threads 64..127 beta.  Rows past the chunk read
// nothing and hold k = q = v = 0, alpha = 1, beta = 0.
struct RawChunk {
    uint4 k[4], q[4], v[4];
    uint16_t a, b;
};

__device__ __forceinline__ void load_chunk(RawChunk &R, const uint16_t *kg, const uint16_t *qg,
                                           const uint16_t *vg, const uint16_t *ag, const uint16_t *bg,
                                           int64_t row_base, int H, int h, int tid, int lc,
                                           bool want_q) {
    const int lrow = tid >> 4;
    const int lcol = 8 * (tid & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 16 * i + lrow;
        if (t < lc) {
            const int64_t rowi = (row_base + t) * H + h;
            R.k[i] = *reinterpret_cast<const uint4 *>(kg + rowi * DK + lcol);
            R.v[i] = *reinterpret_cast<const uint4 *>(vg + rowi * DV + lcol);
            R.q[i] = want_q ? *reinterpret_cast<const uint4 *>(qg + rowi * DK + lcol) : make_uint4(0, 0, 0, 0);
        } else {
            R.k[i] = make_uint4(0, 0, 0, 0);
            R.v[i] = make_uint4(0, 0, 0, 0);
            R.q[i] = make_uint4(0, 0, 0, 0);
        }
    }
    if (tid < C) {
        R.a = tid < lc ? ag[(row_base + tid) * H + h] : (uint16_t)0x3f80;  // alpha = 1
    } else if (tid < 2 * C) {
        const int t = tid - C;
        R.b = t < lc ? bg[(row_base + t) * H + h] : (uint16_t)0;          // beta = 0
    }
}

__global__ __launch_bounds__(NT, 1) void chunked_kernel(const LaunchDesc P)
{
    __shared__ Smem sm;

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int h = L % P.H;
    const int r = L / P.H;
    const int b = P.req[r];
    const int H = P.H;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi32 = lane >> 5;
    const bool want_o = P.o != nullptr;
    const bool norm_q = (P.flags & kNormQ) != 0;

    const uint16_t *kg = static_cast<const uint16_t *>(P.k);
    const uint16_t *qg = static_cast<const uint16_t *>(P.q);
    const uint16_t *vg = static_cast<const uint16_t *>(P.v);
    const uint16_t *ag = static_cast<const uint16_t *>(P.alpha);
    const uint16_t *bg = static_cast<const uint16_t *>(P.beta);
    uint16_t *og = static_cast<uint16_t *>(P.o);

    // ---- state S^T in accumulator layout: tile a covers d_k rows 32a..32a+31,
    // lane holds value row dv = 32w + l32 and d_k rows 8(j/4) + 4*hi32 + j%4.
    floatx16 Sacc[4];
    {
        const int dv = 32 * w + l32;
        if (P.init_off[r] >= 0) {
            const float *src = P.init_base + P.init_off[r] + (int64_t)h * DV * DK + (int64_t)dv * DK;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 v4 = *reinterpret_cast<const float4 *>(src + 32 * a + 8 * q4 + 4 * hi32);
                    Sacc[a][4 * q4 + 0] = v4.x;
                    Sacc[a][4 * q4 + 1] = v4.y;
                    Sacc[a][4 * q4 + 2] = v4.z;
                    Sacc[a][4 * q4 + 3] = v4.w;
                }
        } else {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int j = 0; j < 16; ++j) Sacc[a][j] = 0.f;
        }
    }

    // Zero the upper 16x16 blocks of P inside the two diagonal 32x32 tiles;
    // they are read by the output product and never written afterwards.
    for (int idx = tid; idx < 2 * 16 * 16; idx += NT) {
        const int blk = idx >> 8, e = idx & 255;
        const int t = 32 * blk + (e >> 4), s = 32 * blk + 16 + (e & 15);
        sm.pc[t * TST + s] = (_Float16)0.f;
    }

    const int len = P.len[r];
    const int64_t row0 = P.row0[r];
    int ne = P.emit_begin[r];
    const int ne_end = P.emit_begin[r + 1];


    // ---- raw loads of one chunk into registers: lane covers tokens 16i + tid/16
    // (i = 0..3) and elements 8*(tid%16) .. +7 of q, k and v.
    RawChunk raw;
    raw.a = 0x3f80;
    raw.b = 0;
    const int lrow = tid >> 4;
    const int lcol = 8 * (tid & 15);

    int t0 = 0;
    int lc = len > 0 ? chunk_len(P, len, 0, ne, ne_end) : 0;
    if (len > 0) load_chunk(raw, kg, qg, vg, ag, bg, row0, H, h, tid, lc, want_o);

    while (t0 < len) {
        __syncthreads();  // previous chunk's LDS reads are done

        // ---- phase 1: per-token scales, fp16 operands into LDS ----------------
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * i + lrow;
            float kf[8], qf[8];
            const uint32_t kw[4] = {raw.k[i].x, raw.k[i].y, raw.k[i].z, raw.k[i].w};
            const uint32_t qw[4] = {raw.q[i].x, raw.q[i].y, raw.q[i].z, raw.q[i].w};
            const uint32_t vw[4] = {raw.v[i].x, raw.v[i].y, raw.v[i].z, raw.v[i].w};
            float kss = 0.f, kmx = 0.f, qss = 0.f, qmx = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[2 * e] = __uint_as_float(kw[e] << 16);
                kf[2 * e + 1] = __uint_as_float(kw[e] & 0xffff0000u);
                qf[2 * e] = __uint_as_float(qw[e] << 16);
                qf[2 * e + 1] = __uint_as_float(qw[e] & 0xffff0000u);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kss += kf[e] * kf[e];
                kmx = fmaxf(kmx, fabsf(kf[e]));
                qss += qf[e] * qf[e];
                qmx = fmaxf(qmx, fabsf(qf[e]));
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                kss += __shfl_xor(kss, o);
                qss += __shfl_xor(qss, o);
                kmx = fmaxf(kmx, __shfl_xor(kmx, o));
                qmx = fmaxf(qmx, __shfl_xor(qmx, o));
            }
            int Ek, Eq;
            frexpf(kmx, &Ek);
            frexpf(qmx, &Eq);
            half8 kh, qh;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kh[e] = (_Float16)ldexpf(kf[e], -Ek);
                qh[e] = (_Float16)ldexpf(qf[e], -Eq);
            }
            _Float16 *kp = &sm.kc[t * KST + lcol];
            _Float16 *qp = &sm.qc[t * KST + lcol];
            *reinterpret_cast<half4 *>(kp) = __builtin_shufflevector(kh, kh, 0, 1, 2, 3);
            *reinterpret_cast<half4 *>(kp + 4) = __builtin_shufflevector(kh, kh, 4, 5, 6, 7);
            *reinterpret_cast<half4 *>(qp) = __builtin_shufflevector(qh, qh, 0, 1, 2, 3);
            *reinterpret_cast<half4 *>(qp + 4) = __builtin_shufflevector(qh, qh, 4, 5, 6, 7);
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.kct[(lcol + e) * TST + t] = kh[e];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sm.vct[(lcol + 2 * e) * TST + t] = (uint16_t)(vw[e] & 0xffffu);
                sm.vct[(lcol + 2 * e + 1) * TST + t] = (uint16_t)(vw[e] >> 16);
            }
            if ((tid & 15) == 0) {
                sm.kap[t] = kss > 0.f ? ldexpf(1.f, Ek) / sqrtf(kss) : 0.f;
                sm.kapq[t] = norm_q ? (qss > 0.f ? ldexpf(1.f, Eq) / sqrtf(qss) : 0.f) : ldexpf(1.f, Eq);
            }
        }
        if (tid < C) {
            sm.g[tid] = logf(fmaxf(bf(raw.a), 1e-30f));
        } else if (tid < 2 * C) {
            sm.beta[tid - C] = bf(raw.b);
        }

        // prefetch the next chunk while this one is processed
        const int t0n = t0 + lc;
        int nen = ne;
        if (nen < ne_end && P.emit_after[nen] == t0n) ++nen;
        const int lcn = t0n < len ? chunk_len(P, len, t0n, nen, ne_end) : 0;
        if (lcn > 0) load_chunk(raw, kg, qg, vg, ag, bg, row0 + t0n, H, h, tid, lcn, want_o);

        __syncthreads();

        // ---- phase 2: decay prefix sums (wave 0) and the key/query Gram tiles --
        if (w == 0) {
            float x = sm.g[lane];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(x, o);
                if (lane >= o) x += y;
            }
            const float gC = __shfl(x, 63);
            const float e = expf(x);
            sm.g[lane] = x;
            sm.eg[lane] = e;
            sm.egk[lane] = e * sm.kap[lane];
            sm.wsc[lane] = expf(gC - x) * sm.kap[lane];
            if (lane == 0) sm.egC = expf(gC);
        }
        floatx4 gacc[5];
#pragma unroll
        for (int it = 0; it < 5; ++it) {
            const int item = w + 4 * it;
            const int idx = item % 10;
            const _Float16 *src = item < 10 ? sm.kc : sm.qc;
            const int mt = kTileM[idx], nt = kTileN[idx];
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int c0 = 32 * ks + 8 * (lane >> 4);
                const half8 A = frag_contig(src + (16 * mt + (lane & 15)) * KST + c0);
                const half8 B = frag_contig(sm.kc + (16 * nt + (lane & 15)) * KST + c0);
                acc = mfma16(A, B, acc);
            }
            gacc[it] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 5; ++it) {
            const int item = w + 4 * it;
            const int idx = item % 10;
            const int mt = kTileM[idx], nt = kTileN[idx];
            const int s = 16 * nt + (lane & 15);
            const float gs = sm.g[s], ks_ = sm.kap[s];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * mt + 4 * (lane >> 4) + j;
                const float dec = expf(sm.g[t] - gs);
                if (item < 10) {
                    sm.aws[t * AST + s] = s < t ? sm.beta[t] * dec * sm.kap[t] * ks_ * gacc[it][j] : 0.f;
                } else {
                    sm.pc[t * TST + s] = (_Float16)(s <= t ? dec * ks_ * gacc[it][j] : 0.f);
                }
            }
        }
        __syncthreads();

        // ---- phase 3: T = (I + A)^{-1} in float32 (blocked, in place) ---------
        if (lane < 16) {
            const int bo = 16 * w;
            float x[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                float acc = rr == lane ? 1.f : 0.f;
                const float *arow = &sm.aws[(bo + rr) * AST + bo];
#pragma unroll
                for (int s = 0; s < rr; ++s) acc -= arow[s] * x[s];
                x[rr] = acc;
            }
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) sm.aws[(bo + rr) * AST + bo + lane] = x[rr];
        }
        __syncthreads();
        {   // 32 x 32 blocks: T10 = -T11 A10 T00, for p = 0, 1
            const int p = tid >> 7, e = tid & 127;
            const int rr = e >> 3, cc = 2 * (e & 7);
            const int R1 = 32 * p + 16, C0 = 32 * p;
            float w0 = 0.f, w1 = 0.f;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const float a = sm.aws[(R1 + rr) * AST + C0 + k];
                w0 += a * sm.aws[(C0 + k) * AST + C0 + cc];
                w1 += a * sm.aws[(C0 + k) * AST + C0 + cc + 1];
            }
            sm.wws[p * 16 * 17 + rr * 17 + cc] = w0;
            sm.wws[p * 16 * 17 + rr * 17 + cc + 1] = w1;
            __syncthreads();
            float x0 = 0.f, x1 = 0.f;
            for (int k = 0; k <= rr; ++k) {
                const float t = sm.aws[(R1 + rr) * AST + R1 + k];
                x0 += t * sm.wws[p * 16 * 17 + k * 17 + cc];
                x1 += t * sm.wws[p * 16 * 17 + k * 17 + cc + 1];
            }
            sm.aws[(R1 + rr) * AST + C0 + cc] = -x0;
            sm.aws[(R1 + rr) * AST + C0 + cc + 1] = -x1;
        }
        __syncthreads();
        {   // 64 x 64: T10 = -T11 A10 T00 with 32 x 32 blocks
            const int rr = tid >> 3, cc = 4 * (tid & 7);
            float wv[4] = {0.f, 0.f, 0.f, 0.f};
            for (int k = 0; k < 32; ++k) {
                const float a = sm.aws[(32 + rr) * AST + k];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k >= cc + q) wv[q] += a * sm.aws[k * AST + cc + q];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) sm.wws[rr * 33 + cc + q] = wv[q];
            __syncthreads();
            float xv[4] = {0.f, 0.f, 0.f, 0.f};
            for (int k = 0; k <= rr; ++k) {
                const float t = sm.aws[(32 + rr) * AST + 32 + k];
#pragma unroll
                for (int q = 0; q < 4; ++q) xv[q] += t * sm.wws[k * 33 + cc + q];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) sm.aws[(32 + rr) * AST + cc + q] = -xv[q];
        }
        __syncthreads();
        {   // T -> fp16 with a power-of-two scale
            float mx = 0.f;
#pragma unroll 4
            for (int m = 0; m < 16; ++m) {
                const int idx = tid + NT * m;
                const int t = idx >> 6, s = idx & 63;
                if (s <= t) mx = fmaxf(mx, fabsf(sm.aws[t * AST + s]));
            }
            mx = wave_max(mx);
            if (lane == 0) sm.red[w] = mx;
            __syncthreads();
            mx = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
            const float sc = ldexpf(1.f, fp16_exp(mx));
#pragma unroll 4
            for (int m = 0; m < 16; ++m) {
                const int idx = tid + NT * m;
                const int t = idx >> 6, s = idx & 63;
                sm.tc[t * TST + s] = (_Float16)(s <= t ? sm.aws[t * AST + s] * sc : 0.f);
            }
        }
        __syncthreads();
        const float unT = ldexpf(1.f, -fp16_exp(fmaxf(fmaxf(sm.red[0], sm.red[1]),
                                                       fmaxf(sm.red[2], sm.red[3]))));

        // ---- phase 4: the state chain of wave w (value rows 32w .. 32w+31) ----
        const int dv = 32 * w + l32;
        float smx = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int j = 0; j < 16; ++j) smx = fmaxf(smx, fabsf(Sacc[a][j]));
        const int eS = fp16_exp(wave_max(smx));
        const float scS = ldexpf(1.f, eS), unS = ldexpf(1.f, -eS);
        half8 Sf[4][2];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            Sf[a][0] = to_frag(Sacc[a], 0, scS);
            Sf[a][1] = to_frag(Sacc[a], 1, scS);
        }
        // Y = K' S0'^T and Z = Q' S0'^T (tokens x value rows of this wave)
        floatx16 Y[2], Z[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            floatx16 acc = {}, zacc = {};
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    acc = mfma32(frag_perm(sm.kc, KST, 32 * u + l32, 32 * a + 16 * ks, lane), Sf[a][ks], acc);
                    if (want_o)
                        zacc = mfma32(frag_perm(sm.qc, KST, 32 * u + l32, 32 * a + 16 * ks, lane), Sf[a][ks], zacc);
                }
            Y[u] = acc;
            Z[u] = zacc;
        }
        // B_t = beta_t (v_t - e^{g_t} kap_t S0 k'_t)
        float bmx = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int t = 32 * u + 8 * q4 + 4 * hi32;
                const uint2 v2 = *reinterpret_cast<const uint2 *>(&sm.vct[dv * TST + t]);
                const float4 bt = *reinterpret_cast<const float4 *>(&sm.beta[t]);
                const float4 ek = *reinterpret_cast<const float4 *>(&sm.egk[t]);
                const float vv[4] = {__uint_as_float(v2.x << 16), __uint_as_float(v2.x & 0xffff0000u),
                                     __uint_as_float(v2.y << 16), __uint_as_float(v2.y & 0xffff0000u)};
                const float bb[4] = {bt.x, bt.y, bt.z, bt.w};
                const float ee[4] = {ek.x, ek.y, ek.z, ek.w};
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const float x = bb[j4] * (vv[j4] - ee[j4] * unS * Y[u][4 * q4 + j4]);
                    Y[u][4 * q4 + j4] = x;
                    bmx = fmaxf(bmx, fabsf(x));
                }
            }
        const int eB = fp16_exp(wave_max(bmx));
        const float scB = ldexpf(1.f, eB);
        half8 Bf[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            Bf[u][0] = to_frag(Y[u], 0, scB);
            Bf[u][1] = to_frag(Y[u], 1, scB);
        }
        // U = T B
        floatx16 U[2];
        const float unTB = unT * ldexpf(1.f, -eB);
        float umx = 0.f;
#pragma unroll
        for (int u2 = 0; u2 < 2; ++u2) {
            floatx16 acc = {};
#pragma unroll
            for (int u = 0; u <= u2; ++u)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    acc = mfma32(frag_perm(sm.tc, TST, 32 * u2 + l32, 32 * u + 16 * hf, lane), Bf[u][hf], acc);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                acc[j] *= unTB;
                umx = fmaxf(umx, fabsf(acc[j]));
            }
            U[u2] = acc;
        }
        // outputs o_t = kapq_t (e^{g_t} S0 q'_t + sum_s P_ts u_s)
        if (want_o) {
            const int eU = fp16_exp(wave_max(umx));
            const float scU = ldexpf(1.f, eU), unU = ldexpf(1.f, -eU);
            half8 Uf[2][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                Uf[u][0] = to_frag(U[u], 0, scU);
                Uf[u][1] = to_frag(U[u], 1, scU);
            }
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                floatx16 po = {};
#pragma unroll
                for (int u = 0; u <= u2; ++u)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
                        po = mfma32(frag_perm(sm.pc, TST, 32 * u2 + l32, 32 * u + 16 * hf, lane), Uf[u][hf], po);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int tb = 32 * u2 + 8 * q4 + 4 * hi32;
                    const float4 e4 = *reinterpret_cast<const float4 *>(&sm.eg[tb]);
                    const float4 k4 = *reinterpret_cast<const float4 *>(&sm.kapq[tb]);
                    const float ee[4] = {e4.x, e4.y, e4.z, e4.w};
                    const float kq[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const int t = tb + j4;
                        if (t < lc) {
                            const float ov = kq[j4] * (ee[j4] * unS * Z[u2][4 * q4 + j4] + unU * po[4 * q4 + j4]);
                            og[((row0 + t0 + t) * H + h) * DV + dv] = f32_to_bf16(ov);
                        }
                    }
                }
            }
        }
        // S_C = e^{g_C} S0 + sum_s (e^{g_C - g_s} kap_s u_s) k'_s^T
        float wmx = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int tb = 32 * u + 8 * q4 + 4 * hi32;
                const float4 s4 = *reinterpret_cast<const float4 *>(&sm.wsc[tb]);
                const float ss[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    U[u][4 * q4 + j4] *= ss[j4];
                    wmx = fmaxf(wmx, fabsf(U[u][4 * q4 + j4]));
                }
            }
        const int eW = fp16_exp(wave_max(wmx));
        const float scW = ldexpf(1.f, eW), unW = ldexpf(1.f, -eW);
        half8 Wf[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            Wf[u][0] = to_frag(U[u], 0, scW);
            Wf[u][1] = to_frag(U[u], 1, scW);
        }
        const float pre = sm.egC * scW;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            floatx16 acc = Sacc[a] * pre;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    acc = mfma32(frag_perm(sm.kct, TST, 32 * a + l32, 32 * u + 16 * hf, lane), Wf[u][hf], acc);
            Sacc[a] = acc * unW;
        }

        t0 += lc;
        if (ne < ne_end && P.emit_after[ne] == t0) {
            store_state(P.emit_base + (((int64_t)b * P.M + P.emit_slot[ne]) * H + h) * DV * DK, Sacc, w,
                        l32, hi32);
            ++ne;
        }
        lc = lcn;
    }

    store_state(P.state_out + ((int64_t)b * H + h) * DV * DK, Sacc, w, l32, hi32);
}

}  // namespace

bool chunked_supported(int dk, int dv, Elem e) {
    return dk == DK && dv == DV && e == Elem::BF16;
}

hipError_t launch_chunked(const LaunchDesc &d, int dk, int dv, Elem e, hipStream_t s) {
    if (!chunked_supported(dk, dv, e)) return hipErrorNotSupported;
    const int nwg = d.nreq * d.H;
    if (nwg == 0) return hipSuccess;
    hipLaunchKernelGGL(chunked_kernel, dim3(nwg), dim3(NT), 0, s, d);
    return hipGetLastError();
}

}  // namespace gdn
