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
// Precision: the dense products run on fp16 MFMA (32x32x16, 16x16x32 and
// 16x16x16 shapes) with float32 accumulation.  Keys are unit vectors (the
// fused L2 norm), so |k_i| <= 1 fits fp16 as is; queries are normalised too,
// or scaled per token by an exact power of two.  The state, B, U and T are
// scaled by exact powers of two per wave or per chunk before rounding to
// fp16.  T is built blockwise: 16x16 diagonal blocks by float32 substitution,
// the off-diagonal blocks by two doubling levels on MFMA.  The state itself
// never leaves float32.  Gates are handled in log2 space with the native
// v_exp_f32 / v_log_f32.
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
    _Float16 kc[C * KST];     // unit keys k^, token-major
    _Float16 qc[C * KST];     // q^ (or q / 2^E), token-major
    _Float16 kct[DK * TST];   // unit keys, key-major
    uint16_t vct[DV * TST];   // v (bf16 bits), value-major
    _Float16 tc[C * TST];     // T scaled to fp16
    _Float16 pc[C * TST];     // P_ts = 2^{g_t-g_s} (q'_t . k^_s), s <= t
    float aws[C * AST];       // A, then T, in float32
    float wws[32 * 33];       // scratch for the blocked inverse
    alignas(16) float beta[C];
    alignas(16) float g[C];               // log2 alpha, then its chunk-local prefix sum
    alignas(16) float eg[C];              // 2^{g_t}
    alignas(16) float kapq[C];            // 1, or 2^E_t for unnormalised queries
    alignas(16) float wsc[C];             // 2^{g_C - g_t}
    float red[NW];
    float egC;
};

// Workgroup barrier that orders LDS traffic only: outstanding global loads
// (the next chunk's prefetch) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_(float x) { return __builtin_amdgcn_logf(x); }

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

// v_mfma_f32_16x16x16_f16: lane i holds A[i%16][4(i/16)+j] and B[4(i/16)+j][i%16];
// its result D[4(i/16)+j][i%16] is laid out like a B operand.
__device__ __forceinline__ floatx4 mfma1616(half4 a, half4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// A operand of mfma1616 from a float32 row-major block (rows r0.., cols c0..).
__device__ __forceinline__ half4 a1616(const float *m, int stride, int r0, int c0, int lane) {
    const float4 v = *reinterpret_cast<const float4 *>(m + (r0 + (lane & 15)) * stride + c0 + 4 * (lane >> 4));
    half4 h;
    h[0] = (_Float16)v.x; h[1] = (_Float16)v.y; h[2] = (_Float16)v.z; h[3] = (_Float16)v.w;
    return h;
}

// B operand of mfma1616 from a float32 row-major block.
__device__ __forceinline__ half4 b1616(const float *m, int stride, int r0, int c0, int lane) {
    const float *p = m + (r0 + 4 * (lane >> 4)) * stride + c0 + (lane & 15);
    half4 h;
    h[0] = (_Float16)p[0]; h[1] = (_Float16)p[stride]; h[2] = (_Float16)p[2 * stride]; h[3] = (_Float16)p[3 * stride];
    return h;
}

// Lower-triangular 16x16 tiles (mt, nt), nt <= mt, of a 64 x 64 matrix,
// enumerated 0..9 and packed 4 bits per entry (no memory lookup).
__device__ __forceinline__ int tile_m(int idx) { return (int)((0x3333222110ull >> (4 * idx)) & 0xf); }
__device__ __forceinline__ int tile_n(int idx) { return (int)((0x3210210100ull >> (4 * idx)) & 0xf); }


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

// Raw bf16 rows of the next chunk, staged in LDS by direct global->LDS loads
// (global_load_lds_dwordx4), so the prefetch holds no VGPRs and stays in
// flight across LDS-only barriers.  Rows are 256 B, row-major.  The gates
// (one bf16 per token) go through a register instead: a sub-dword LDS DMA
// still writes one dword per lane.
struct RawStage {
    uint16_t k[C * DK];
    uint16_t q[C * DK];
    uint16_t v[C * DV];
};

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

// Lane l of the wave copies `size` bytes from g to (LDS base) + l * size.
__device__ __forceinline__ void dma16(const void *g, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds((gvoid_t *)g, (lvoid_t *)lds_wave_base, 16, 0, 0);
}

// Queue the loads of one chunk of lc tokens starting at packed row row_base.
// Wave w, step i copies rows 16 i + 4 w .. +3 (lane l: row + l/16, 16 B at
// column 8 (l%16)); wave 0 loads alpha and wave 1 beta into `gate` (issued
// first, so waiting for it leaves the copies in flight).  Rows at or past lc
// are not read; the consumer treats them as k = q = v = 0, alpha = 1, beta = 0.
__device__ __forceinline__ void dma_chunk(RawStage &R, uint16_t &gate, const uint16_t *kg,
                                          const uint16_t *qg, const uint16_t *vg, const uint16_t *ag,
                                          const uint16_t *bg, int64_t row_base, int H, int h, int w,
                                          int lane, int lc, bool want_q) {
    if (w < 2 && lane < lc) gate = (w == 0 ? ag : bg)[(row_base + lane) * H + h];
    const int sub = lane >> 4;
    const int col = 8 * (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r0 = 16 * i + 4 * w;
        if (r0 + sub < lc) {
            const int64_t rowi = (row_base + r0 + sub) * H + h;
            dma16(kg + rowi * DK + col, &R.k[r0 * DK]);
            dma16(vg + rowi * DV + col, &R.v[r0 * DV]);
            if (want_q) dma16(qg + rowi * DK + col, &R.q[r0 * DK]);
        }
    }
}

// Wait for this wave's outstanding loads (the staged chunk), then barrier.
__device__ __forceinline__ void vm_lds_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ __launch_bounds__(NT, 1) void chunked_kernel(const LaunchDesc P)
{
    __shared__ Smem sm;
    __shared__ RawStage sraw;

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int h = L % P.H;
    const int r = L / P.H;
    const int b = P.req[r];
    const int H = P.H;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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
    const int lrow = tid >> 4;
    const int lcol = 8 * (tid & 15);

    int t0 = 0;
    int lc = len > 0 ? chunk_len(P, len, 0, ne, ne_end) : 0;
    uint16_t gate = 0;
    if (len > 0) dma_chunk(sraw, gate, kg, qg, vg, ag, bg, row0, H, h, w, lane, lc, want_o);

    while (t0 < len) {
        vm_lds_barrier();  // staged chunk has landed; previous chunk's LDS reads are done

        // ---- phase 1: unit keys / queries as fp16 operands into LDS ----------
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * i + lrow;
            float kf[8], qf[8];
            const bool live = t < lc;
            const uint4 z4 = make_uint4(0, 0, 0, 0);
            const uint4 rk = live ? *reinterpret_cast<const uint4 *>(&sraw.k[t * DK + lcol]) : z4;
            const uint4 rq = (live && want_o) ? *reinterpret_cast<const uint4 *>(&sraw.q[t * DK + lcol]) : z4;
            const uint4 rv = live ? *reinterpret_cast<const uint4 *>(&sraw.v[t * DV + lcol]) : z4;
            const uint32_t kw[4] = {rk.x, rk.y, rk.z, rk.w};
            const uint32_t qw[4] = {rq.x, rq.y, rq.z, rq.w};
            const uint32_t vw[4] = {rv.x, rv.y, rv.z, rv.w};
            float kss = 0.f, qss = 0.f, qmx = 0.f;
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
                qss += qf[e] * qf[e];
                qmx = fmaxf(qmx, fabsf(qf[e]));
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                kss += __shfl_xor(kss, o);
                qss += __shfl_xor(qss, o);
                if (!norm_q) qmx = fmaxf(qmx, __shfl_xor(qmx, o));
            }
            // k^ = k / ||k|| (a zero key stays zero); q^ likewise, or q / 2^E
            const float ks = kss > 0.f ? rsqrtf(kss) : 0.f;
            int Eq = 0;
            if (!norm_q) frexpf(qmx, &Eq);
            const float qs = norm_q ? (qss > 0.f ? rsqrtf(qss) : 0.f) : ldexpf(1.f, -Eq);
            half8 kh, qh;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kh[e] = (_Float16)(kf[e] * ks);
                qh[e] = (_Float16)(qf[e] * qs);
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
            if ((tid & 15) == 0) sm.kapq[t] = norm_q ? 1.f : ldexpf(1.f, Eq);
        }
        if (tid < C) {
            sm.g[tid] = tid < lc ? log2_(fmaxf(bf(gate), 1e-30f)) : 0.f;
        } else if (tid < 2 * C) {
            sm.beta[tid - C] = tid - C < lc ? bf(gate) : 0.f;
        }
        lds_barrier();

        // ---- phase 2: decay prefix sums (wave 0) and the key/query Gram tiles --
        if (w == 0) {
            float x = sm.g[lane];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(x, o);
                if (lane >= o) x += y;
            }
            const float gC = __shfl(x, 63);
            sm.g[lane] = x;
            sm.eg[lane] = exp2_(x);
            sm.wsc[lane] = exp2_(gC - x);
            if (lane == 0) sm.egC = exp2_(gC);
        }
        floatx4 gacc[5];
#pragma unroll
        for (int it = 0; it < 5; ++it) {
            const int item = w + 4 * it;
            const int idx = item % 10;
            const _Float16 *src = item < 10 ? sm.kc : sm.qc;
            const int mt = tile_m(idx), nt = tile_n(idx);
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
        lds_barrier();
#pragma unroll
        for (int it = 0; it < 5; ++it) {
            const int item = w + 4 * it;
            const int idx = item % 10;
            const int mt = tile_m(idx), nt = tile_n(idx);
            const int s = 16 * nt + (lane & 15);
            const float gs = sm.g[s];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * mt + 4 * (lane >> 4) + j;
                const float dec = exp2_(sm.g[t] - gs);
                if (item < 10) {
                    sm.aws[t * AST + s] = s < t ? sm.beta[t] * dec * gacc[it][j] : 0.f;
                } else {
                    sm.pc[t * TST + s] = (_Float16)(s <= t ? dec * gacc[it][j] : 0.f);
                }
            }
        }
        lds_barrier();

        // ---- phase 3: T = (I + A)^{-1} (blocked, in place in aws) -------------
        // 16 x 16 diagonal blocks: forward substitution in float32, one column per lane
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
        lds_barrier();
        // 32 x 32 blocks p = 0, 1: T10 = -T11 (A10 T00), waves 0 and 1
        if (w < 2) {
            const int R1 = 32 * w + 16, C0 = 32 * w;
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
            const floatx4 W4 = mfma1616(a1616(sm.aws, AST, R1, C0, lane), b1616(sm.aws, AST, C0, C0, lane), z4);
            half4 wf;
#pragma unroll
            for (int j = 0; j < 4; ++j) wf[j] = (_Float16)W4[j];
            const floatx4 X4 = mfma1616(a1616(sm.aws, AST, R1, R1, lane), wf, z4);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm.aws[(R1 + 4 * (lane >> 4) + j) * AST + C0 + (lane & 15)] = -X4[j];
        }
        lds_barrier();
        // 64 x 64: T10 = -T11 (A10 T00) with 32 x 32 blocks; wave w owns the
        // 16 x 16 output block (rb, cb) = (w / 2, w % 2)
        {
            const int rb = w >> 1, cb = w & 1;
            floatx4 W4 = {0.f, 0.f, 0.f, 0.f};
            for (int kb = cb; kb < 2; ++kb)
                W4 = mfma1616(a1616(sm.aws, AST, 32 + 16 * rb, 16 * kb, lane),
                              b1616(sm.aws, AST, 16 * kb, 16 * cb, lane), W4);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm.wws[(16 * rb + 4 * (lane >> 4) + j) * 33 + 16 * cb + (lane & 15)] = W4[j];
            lds_barrier();
            floatx4 X4 = {0.f, 0.f, 0.f, 0.f};
            for (int kb = 0; kb <= rb; ++kb)
                X4 = mfma1616(a1616(sm.aws, AST, 32 + 16 * rb, 32 + 16 * kb, lane),
                              b1616(sm.wws, 33, 16 * kb, 16 * cb, lane), X4);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm.aws[(32 + 16 * rb + 4 * (lane >> 4) + j) * AST + 16 * cb + (lane & 15)] = -X4[j];
        }
        lds_barrier();
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
            lds_barrier();
            mx = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
            const float sc = ldexpf(1.f, fp16_exp(mx));
#pragma unroll 4
            for (int m = 0; m < 16; ++m) {
                const int idx = tid + NT * m;
                const int t = idx >> 6, s = idx & 63;
                sm.tc[t * TST + s] = (_Float16)(s <= t ? sm.aws[t * AST + s] * sc : 0.f);
            }
        }
        lds_barrier();
        const float unT = ldexpf(1.f, -fp16_exp(fmaxf(fmaxf(sm.red[0], sm.red[1]),
                                                       fmaxf(sm.red[2], sm.red[3]))));

        // The staging area was consumed in phase 1: queue the next chunk now, so
        // that its copies overlap the state chain (queued any earlier, LDS reads
        // of phase 3 would have to wait for them).
        const int t0n = t0 + lc;
        int nen = ne;
        if (nen < ne_end && P.emit_after[nen] == t0n) ++nen;
        const int lcn = t0n < len ? chunk_len(P, len, t0n, nen, ne_end) : 0;
        if (lcn > 0) dma_chunk(sraw, gate, kg, qg, vg, ag, bg, row0 + t0n, H, h, w, lane, lcn, want_o);

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
        // Y = K^ S0'^T and Z = Q' S0'^T (tokens x value rows of this wave)
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
        // B_t = beta_t (v_t - 2^{g_t} S0 k^_t)
        float bmx = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int t = 32 * u + 8 * q4 + 4 * hi32;
                const uint2 v2 = *reinterpret_cast<const uint2 *>(&sm.vct[dv * TST + t]);
                const float4 bt = *reinterpret_cast<const float4 *>(&sm.beta[t]);
                const float4 ek = *reinterpret_cast<const float4 *>(&sm.eg[t]);
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
        // outputs o_t = kapq_t (2^{g_t} S0 q'_t + sum_s P_ts u_s)
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
        // S_C = 2^{g_C} S0 + sum_s (2^{g_C - g_s} u_s) k^_s^T
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
