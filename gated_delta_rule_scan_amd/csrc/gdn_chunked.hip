// Chunked matrix-core replay kernel for gfx950: bf16 inputs, float32 state,
// d_k = d_v = 128, unit (normalised) keys.
//
// The recurrence of "Tail-Replay: Escaping the Curse of Linear Attention in
// Prefix Caching for Hybrid LLMs" §2.3 eq. (1) (state d_v x d_k, key operator
// on the right) is advanced C = 32 tokens at a time.  Inside a chunk, with
// g_t = sum_{i<=t} log2 alpha_i (chunk-local) and u_t = beta_t (v_t - alpha_t
// S_{t-1} k_t), unrolling eq. (1) gives
//     S_t = 2^{g_t} S_0 + sum_{s<=t} 2^{g_t - g_s} u_s k_s^T,
// and the u_t solve a unit lower-triangular system
//     (I + A) U = B,  A_ts = beta_t 2^{g_t - g_s} (k_t . k_s)  (s < t),
//                     B_t  = beta_t (v_t - 2^{g_t} S_0 k_t),
// so that, with T = (I + A)^{-1} (it depends on keys and gates only):
//     U   = T B
//     o_t = 2^{g_t} S_0 q_t + sum_{s<=t} 2^{g_t - g_s} (q_t . k_s) u_s
//     S_C = 2^{g_C} S_0 + sum_s 2^{g_C - g_s} u_s k_s^T.
// This is the compact-WY way of applying a product of rank-1 modifications of
// the identity (Golub & Van Loan, Matrix Computations, §5.1) to the chunk.
//
// Precision: the dense products run on fp16 MFMA with float32 accumulation.
// Keys are unit vectors (|k_i| <= 1 fits fp16 as is); queries are normalised
// too, or scaled per token by an exact power of two.  The state, B, U and T
// are scaled by exact powers of two before rounding to fp16.  T is formed
// blockwise: the two 16 x 16 diagonal blocks by float32 substitution, the
// off-diagonal block by one doubling step on MFMA.  The state itself never
// leaves float32; it is held as S = 2^sig * Sacc with a per-wave exponent sig,
// so that each chunk rescales it once.
//
// Work split: one workgroup of 4 waves per (request, head), two workgroups per
// CU (LDS ~70 KB each).  Wave w owns value rows [32w, 32w + 32).  The state is
// kept transposed, S^T (d_k x d_v), in MFMA accumulator layout; because the
// reduction index of an MFMA may be permuted freely (as long as both operands
// agree), each wave feeds its own accumulators back as B fragments of the
// next chunk's products, so a wave's chunk-to-chunk chain never touches LDS
// for the state.  Wave 0 also forms T while the other waves start the
// state-dependent products.  The next chunk's q/k/v rows are copied into LDS
// with global_load_lds_dwordx4 while the current chunk runs.
#include "gdn_launch.h"
#include "gdn_numeric.h"

namespace gdn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int C = 32;        // tokens per chunk
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int NW = 4;        // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int KST = DK + 4;  // row stride (halves) of kc / qc
constexpr int TST = C + 4;   // row stride (halves) of kct / vct / tc / pc
constexpr int AST = C + 4;   // row stride (floats) of aws

struct Smem {
    alignas(16) uint16_t rk[C * DK];   // raw bf16 rows of the next chunk (LDS DMA)
    alignas(16) uint16_t rq[C * DK];
    alignas(16) uint16_t rv[C * DV];
    alignas(16) _Float16 kc[C * KST];  // unit keys, token-major
    alignas(16) _Float16 qc[C * KST];  // q^ (or q / 2^E), token-major
    alignas(16) _Float16 kct[DK * TST];  // unit keys, key-major
    alignas(16) uint16_t vct[DV * TST];  // v (bf16 bits), value-major; then o staging
    alignas(16) _Float16 tc[C * TST];  // T scaled to fp16
    alignas(16) _Float16 pc[C * TST];  // P_ts = 2^{g_t - g_s} (q'_t . k_s), s <= t
    alignas(16) float aws[C * AST];    // A, then T, in float32
    alignas(16) float atd[2 * 16 * 16];  // diagonal 16x16 blocks of A, transposed
    alignas(16) float beta[C];
    alignas(16) float g[C];            // log2 alpha, then its chunk-local prefix sum
    alignas(16) float eg[C];           // 2^{g_t}
    alignas(16) float wsc[C];          // 2^{g_C - g_t}
    alignas(16) float kapq[C];         // 1, or 2^E_t for unnormalised queries
    float unT;
};

// Workgroup barrier ordering LDS traffic only: outstanding global loads
// (the next chunk's copies) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Wait for this wave's outstanding loads (the staged chunk), then barrier.
__device__ __forceinline__ void vm_lds_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_(float x) { return __builtin_amdgcn_logf(x); }

// Cross-lane steps on the VALU (DPP) rather than through LDS.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWMASK,
                                                                  0xf, true));
}
// Sum / max over each row of 16 lanes; every lane gets its row's result.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0x140>(x);  // row_mirror
    return x;
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0x140>(x));
    return x;
}
__device__ __forceinline__ float lane_val(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// Maximum over the wave, as a wave-uniform value (all lanes must be active).
__device__ __forceinline__ float wave_max(float x) {
    x = row16_max(x);
    return fmaxf(fmaxf(lane_val(x, 0), lane_val(x, 16)), fmaxf(lane_val(x, 32), lane_val(x, 48)));
}
// Inclusive prefix sum over lanes 0..31 (row_shr within rows, then row_bcast:15).
__device__ __forceinline__ float scan32(float x) {
    x += dpp<0x111>(x);
    x += dpp<0x112>(x);
    x += dpp<0x114>(x);
    x += dpp<0x118>(x);
    x += dpp<0x142, 0xa>(x);
    return x;
}

// Power-of-two exponent e bringing max|x| into [2^14, 2^15) (x * 2^e fits fp16).
__device__ __forceinline__ int fp16_exp(float mx) {
    int E;
    frexpf(mx, &E);
    return 15 - E;
}

__device__ __forceinline__ float bf(uint16_t b) { return bf16_to_f32(b); }

__device__ __forceinline__ half4 ld4(const _Float16 *p) {
    return *reinterpret_cast<const half4 *>(p);
}

// A fragment of v_mfma_f32_32x32x16_f16 from a row-major fp16 tile with the
// reduction index permuted: lane i takes row `row`, columns
// c0 + 4*(i/32) + {0..3} and c0 + 8 + 4*(i/32) + {0..3}.  This matches the
// order in which a 32 x 32 accumulator holds its rows (see to_frag).
__device__ __forceinline__ half8 frag_perm(const _Float16 *base, int stride, int row, int c0, int lane) {
    const _Float16 *p = base + row * stride + c0 + 4 * (lane >> 5);
    const half4 lo = ld4(p), hi = ld4(p + 8);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ half8 frag_contig(const _Float16 *p) {
    const half4 lo = ld4(p), hi = ld4(p + 4);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Slots 8*hf .. 8*hf+7 of a 32x32 accumulator, scaled, as an fp16 B fragment.
__device__ __forceinline__ half8 to_frag(const floatx16 &acc, int hf, float scale) {
    half8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (_Float16)(acc[8 * hf + j] * scale);
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

typedef __attribute__((address_space(3))) void lvoid_t;

// Lane l of the wave copies 16 bytes from base + voff (bytes) to
// (LDS base) + 16 l (global_load_lds_dwordx4 with an SGPR base; the LDS base
// goes in M0).  Issued as inline assembly so that the compiler does not order
// later LDS reads of other buffers behind it: the only wait for these copies
// is the explicit vmcnt(0) at the top of the next chunk.
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void dma16(uint64_t base, uint32_t voff, void *lds_wave_base) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)reinterpret_cast<uintptr_t>((lvoid_t *)lds_wave_base));
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

// Chunk schedule: up to C tokens, cut at the next emission position.
__device__ __forceinline__ int chunk_len(const LaunchDesc &P, int len, int t0, int e, int e_end) {
    int lc = min(C, len - t0);
    if (e < e_end) lc = min(lc, P.emit_after[e] - t0);
    return lc;
}

// Queue the loads of one chunk of lc tokens starting at packed row row_base.
// Wave w, step i copies rows 16 i + 4 w .. +3 (lane l: row + l/16, 16 B at
// column 8 (l%16)); wave 0 loads alpha and wave 1 beta into `gate` first (a
// sub-dword LDS copy would still write a dword per lane).  Rows at or past lc
// are not read; the consumer treats them as k = q = v = 0, alpha = 1, beta = 0.
__device__ __forceinline__ void dma_chunk(Smem &sm, uint16_t &gate, const uint16_t *kg,
                                          const uint16_t *qg, const uint16_t *vg, const uint16_t *ag,
                                          const uint16_t *bg, int64_t row_base, int H, int h, int w,
                                          int lane, int lc, bool want_q) {
    if (w < 2 && lane < lc) gate = (w == 0 ? ag : bg)[(row_base + lane) * H + h];
    const int sub = lane >> 4;
    const int64_t e0 = (row_base * H + h) * DK;  // element offset of the chunk's first row
    const uint64_t kb = uniform64(reinterpret_cast<uint64_t>(kg + e0));
    const uint64_t qb = uniform64(reinterpret_cast<uint64_t>(qg + e0));
    const uint64_t vb = uniform64(reinterpret_cast<uint64_t>(vg + e0));
#pragma unroll
    for (int i = 0; i < C / 16; ++i) {
        const int r0 = 16 * i + 4 * w;
        if (r0 + sub < lc) {
            const uint32_t off = (uint32_t)(((r0 + sub) * H * DK + 8 * (lane & 15)) * 2);
            dma16(kb, off, &sm.rk[r0 * DK]);
            dma16(vb, off, &sm.rv[r0 * DV]);
            if (want_q) dma16(qb, off, &sm.rq[r0 * DK]);
        }
    }
}

// Store S = 2^sig * Sacc (held as S^T tiles) to a d_v x d_k row-major block.
__device__ __forceinline__ void store_state(float *dst_head, const floatx16 (&Sacc)[4], int sig, int w,
                                            int l32, int hi32) {
    float *dst = dst_head + (int64_t)(32 * w + l32) * DK;
    const float sc = ldexpf(1.f, sig);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<float4 *>(dst + 32 * a + 8 * q4 + 4 * hi32) =
                make_float4(Sacc[a][4 * q4] * sc, Sacc[a][4 * q4 + 1] * sc, Sacc[a][4 * q4 + 2] * sc,
                            Sacc[a][4 * q4 + 3] * sc);
}

__global__ __launch_bounds__(NT, 2) void chunked_kernel(const LaunchDesc P)
{
    __shared__ Smem sm;

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
    const int dv = 32 * w + l32;
    const bool want_o = P.o != nullptr;
    const bool norm_q = (P.flags & kNormQ) != 0;

    const uint16_t *kg = static_cast<const uint16_t *>(P.k);
    const uint16_t *qg = static_cast<const uint16_t *>(P.q);
    const uint16_t *vg = static_cast<const uint16_t *>(P.v);
    const uint16_t *ag = static_cast<const uint16_t *>(P.alpha);
    const uint16_t *bg = static_cast<const uint16_t *>(P.beta);
    uint16_t *og = static_cast<uint16_t *>(P.o);

    // ---- state S^T = 2^sig * Sacc: tile a covers d_k rows 32a..32a+31; the
    // lane holds value row dv and d_k rows 8(j/4) + 4*hi32 + j%4 of each tile.
    floatx16 Sacc[4];
    int sig = 0;
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

    // The upper-right 16x16 blocks of P and T are read by the products and
    // never written.
    for (int idx = tid; idx < 16 * 16; idx += NT) {
        sm.pc[(idx >> 4) * TST + 16 + (idx & 15)] = (_Float16)0.f;
        sm.tc[(idx >> 4) * TST + 16 + (idx & 15)] = (_Float16)0.f;
    }

    const int len = P.len[r];
    const int64_t row0 = P.row0[r];
    int ne = P.emit_begin[r];
    const int ne_end = P.emit_begin[r + 1];
    const int lrow = tid >> 4;
    const int lcol = 8 * (tid & 15);

    int t0 = 0;
    int lc = len > 0 ? chunk_len(P, len, 0, ne, ne_end) : 0;
    uint16_t gate = 0;
    if (len > 0) dma_chunk(sm, gate, kg, qg, vg, ag, bg, row0, H, h, w, lane, lc, want_o);

    while (t0 < len) {
        vm_lds_barrier();  // staged chunk has landed; the previous chunk's LDS reads are done

        // ---- phase 1: unit keys / queries as fp16 operands, v transposed -------
#pragma unroll
        for (int i = 0; i < C / 16; ++i) {
            const int t = 16 * i + lrow;
            const bool live = t < lc;
            const uint4 z4 = make_uint4(0, 0, 0, 0);
            const uint4 rk = live ? *reinterpret_cast<const uint4 *>(&sm.rk[t * DK + lcol]) : z4;
            const uint4 rq = (live && want_o) ? *reinterpret_cast<const uint4 *>(&sm.rq[t * DK + lcol]) : z4;
            const uint4 rv = live ? *reinterpret_cast<const uint4 *>(&sm.rv[t * DV + lcol]) : z4;
            const uint32_t kw[4] = {rk.x, rk.y, rk.z, rk.w};
            const uint32_t qw[4] = {rq.x, rq.y, rq.z, rq.w};
            const uint32_t vw[4] = {rv.x, rv.y, rv.z, rv.w};
            float kf[8], qf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[2 * e] = __uint_as_float(kw[e] << 16);
                kf[2 * e + 1] = __uint_as_float(kw[e] & 0xffff0000u);
                qf[2 * e] = __uint_as_float(qw[e] << 16);
                qf[2 * e + 1] = __uint_as_float(qw[e] & 0xffff0000u);
            }
            float kss = 0.f, qss = 0.f, qmx = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kss += kf[e] * kf[e];
                qss += qf[e] * qf[e];
                qmx = fmaxf(qmx, fabsf(qf[e]));
            }
            kss = row16_sum(kss);  // one token row per 16 lanes
            qss = row16_sum(qss);
            if (!norm_q) qmx = row16_max(qmx);
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
        } else if (tid >= 64 && tid < 64 + C) {
            sm.beta[tid - 64] = tid - 64 < lc ? bf(gate) : 0.f;
        }
        lds_barrier();

        // ---- phase 2: gate prefix sums and the Gram tiles ----------------------
        // every wave forms g_t (lane t) itself; wave 0 publishes it for phase 4
        const float gscan = scan32(lane < C ? sm.g[lane] : 0.f);
        const float gC = lane_val(gscan, C - 1);
        const float egC = exp2_(gC);
        // items: G = K^K^T tiles (0,0), (1,0), (1,1), then Q'K^T tiles; wave w
        // takes items w and w + 4
        floatx4 gacc[2];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int item = w + 4 * it;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            if (item < 6) {
                const int idx = item % 3;
                const int mt = idx > 0 ? 1 : 0, nt = idx == 2 ? 1 : 0;
                const _Float16 *src = item < 3 ? sm.kc : sm.qc;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int c0 = 32 * ks + 8 * (lane >> 4);
                    acc = mfma16(frag_contig(src + (16 * mt + (lane & 15)) * KST + c0),
                                 frag_contig(sm.kc + (16 * nt + (lane & 15)) * KST + c0), acc);
                }
            }
            gacc[it] = acc;
        }
        if (w == 0 && lane < C) {
            sm.eg[lane] = exp2_(gscan);
            sm.wsc[lane] = exp2_(gC - gscan);
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int item = w + 4 * it;
            if (item < 6) {
                const int idx = item % 3;
                const int mt = idx > 0 ? 1 : 0, nt = idx == 2 ? 1 : 0;
                const int s = 16 * nt + (lane & 15);
                const float gs = __shfl(gscan, s);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = 16 * mt + 4 * (lane >> 4) + j;
                    const float dec = exp2_(__shfl(gscan, t) - gs);
                    if (item < 3) {
                        const float a = s < t ? sm.beta[t] * dec * gacc[it][j] : 0.f;
                        sm.aws[t * AST + s] = a;
                        if (mt == nt) sm.atd[(16 * mt + (s & 15)) * 16 + (t & 15)] = a;
                    } else {
                        sm.pc[t * TST + s] = (_Float16)(s <= t ? dec * gacc[it][j] : 0.f);
                    }
                }
            }
        }
        lds_barrier();

        // ---- phase 3 (wave 0): T = (I + A)^{-1} -> fp16 -------------------------
        if (w == 0) {
            // diagonal blocks (lanes 0..31: block lane/16, column lane%16) by
            // column-oriented substitution: once x_s is final, subtract its
            // multiple from the remaining rows (dependency chain of 16 steps)
            const int bo = 16 * (lane >> 4), c = lane & 15;
            float x[16];
            if (lane < 32) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) x[rr] = rr == c ? 1.f : 0.f;
                const float *at = &sm.atd[bo * 16];
#pragma unroll
                for (int s2 = 0; s2 < 15; ++s2)
#pragma unroll
                    for (int rr = s2 + 1; rr < 16; ++rr) x[rr] -= at[s2 * 16 + rr] * x[s2];
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) sm.aws[(bo + rr) * AST + bo + c] = x[rr];
            }
            // off-diagonal block: T10 = -T11 (A10 T00)
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
            const floatx4 W4 = mfma1616(a1616(sm.aws, AST, 16, 0, lane), b1616(sm.aws, AST, 0, 0, lane), z4);
            half4 wf;
#pragma unroll
            for (int j = 0; j < 4; ++j) wf[j] = (_Float16)W4[j];
            const floatx4 X4 = mfma1616(a1616(sm.aws, AST, 16, 16, lane), wf, z4);
            // fp16 copy with a power-of-two scale, straight from registers
            float mx = fmaxf(fmaxf(fabsf(X4[0]), fabsf(X4[1])), fmaxf(fabsf(X4[2]), fabsf(X4[3])));
            if (lane < 32) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, fabsf(x[rr]));
            }
            const int eT = fp16_exp(wave_max(mx));
            const float sc = ldexpf(1.f, eT);
            if (lane < 32) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) sm.tc[(bo + rr) * TST + bo + c] = (_Float16)(x[rr] * sc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm.tc[(16 + 4 * (lane >> 4) + j) * TST + (lane & 15)] = (_Float16)(-X4[j] * sc);
            if (lane == 0) sm.unT = ldexpf(1.f, -eT);
        }

        // ---- phase 4a: state-dependent products of wave w ----------------------
        float smx = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int j = 0; j < 16; ++j) smx = fmaxf(smx, fabsf(Sacc[a][j]));
        const int eS = fp16_exp(wave_max(smx));
        const float scS = ldexpf(1.f, eS);
        const float unS = ldexpf(1.f, sig - eS);  // S = unS * (fp16 copy)
        floatx16 Y = {}, Z = {};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const half8 sf = to_frag(Sacc[a], ks, scS);
                Y = mfma32(frag_perm(sm.kc, KST, l32, 32 * a + 16 * ks, lane), sf, Y);
                if (want_o) Z = mfma32(frag_perm(sm.qc, KST, l32, 32 * a + 16 * ks, lane), sf, Z);
            }
        // B_t = beta_t (v_t - 2^{g_t} S0 k^_t), in place in Y
        float bmx = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int tb = 8 * q4 + 4 * hi32;
            const uint2 v2 = *reinterpret_cast<const uint2 *>(&sm.vct[dv * TST + tb]);
            const float4 bt = *reinterpret_cast<const float4 *>(&sm.beta[tb]);
            const float4 e4 = *reinterpret_cast<const float4 *>(&sm.eg[tb]);
            const float vv[4] = {__uint_as_float(v2.x << 16), __uint_as_float(v2.x & 0xffff0000u),
                                 __uint_as_float(v2.y << 16), __uint_as_float(v2.y & 0xffff0000u)};
            const float bb[4] = {bt.x, bt.y, bt.z, bt.w};
            const float ee[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const float x = bb[j4] * (vv[j4] - ee[j4] * unS * Y[4 * q4 + j4]);
                Y[4 * q4 + j4] = x;
                bmx = fmaxf(bmx, fabsf(x));
            }
        }
        const int eB = fp16_exp(wave_max(bmx));
        const half8 Bf0 = to_frag(Y, 0, ldexpf(1.f, eB));
        const half8 Bf1 = to_frag(Y, 1, ldexpf(1.f, eB));

        lds_barrier();  // T is ready

        // The staging area was consumed in phase 1: queue the next chunk now so
        // its copies overlap the rest of this chunk.
        const int t0n = t0 + lc;
        int nen = ne;
        if (nen < ne_end && P.emit_after[nen] == t0n) ++nen;
        const int lcn = t0n < len ? chunk_len(P, len, t0n, nen, ne_end) : 0;
        if (lcn > 0) dma_chunk(sm, gate, kg, qg, vg, ag, bg, row0 + t0n, H, h, w, lane, lcn, want_o);

        // ---- phase 4b: U = T B, outputs, state update ---------------------------
        floatx16 U = {};
        U = mfma32(frag_perm(sm.tc, TST, l32, 0, lane), Bf0, U);
        U = mfma32(frag_perm(sm.tc, TST, l32, 16, lane), Bf1, U);
        const float unTB = sm.unT * ldexpf(1.f, -eB);
        float umx = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            U[j] *= unTB;
            umx = fmaxf(umx, fabsf(U[j]));
        }
        if (want_o) {
            // o_t = kapq_t (2^{g_t} S0 q'_t + sum_s P_ts u_s), staged in this wave's
            // rows of vct (its v values are consumed) and stored 16 B per lane
            const int eU = fp16_exp(wave_max(umx));
            const float scU = ldexpf(1.f, eU), unU = ldexpf(1.f, -eU);
            floatx16 po = {};
            po = mfma32(frag_perm(sm.pc, TST, l32, 0, lane), to_frag(U, 0, scU), po);
            po = mfma32(frag_perm(sm.pc, TST, l32, 16, lane), to_frag(U, 1, scU), po);
            uint16_t *stage = &sm.vct[32 * w * TST];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int tb = 8 * q4 + 4 * hi32;
                const float4 e4 = *reinterpret_cast<const float4 *>(&sm.eg[tb]);
                const float4 k4 = *reinterpret_cast<const float4 *>(&sm.kapq[tb]);
                const float ee[4] = {e4.x, e4.y, e4.z, e4.w};
                const float kq[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const float ov = kq[j4] * (ee[j4] * unS * Z[4 * q4 + j4] + unU * po[4 * q4 + j4]);
                    stage[(tb + j4) * 32 + l32] = __builtin_bit_cast(uint16_t, (__bf16)ov);
                }
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int seg = lane + 64 * m;
                const int t = seg >> 2, c8 = 8 * (seg & 3);
                if (t < lc) {
                    const uint4 o4 = *reinterpret_cast<const uint4 *>(&stage[t * 32 + c8]);
                    *reinterpret_cast<uint4 *>(og + ((row0 + t0 + t) * H + h) * DV + 32 * w + c8) = o4;
                }
            }
        }
        // S_C = 2^{g_C} S0 + sum_s (2^{g_C - g_s} u_s) k^_s^T.  With W = wsc * U
        // scaled by 2^eW into fp16, the new representation is sig' = -eW:
        // Sacc' = 2^{g_C} 2^{sig + eW} Sacc + K^T W'.
        float wmx = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int tb = 8 * q4 + 4 * hi32;
            const float4 s4 = *reinterpret_cast<const float4 *>(&sm.wsc[tb]);
            const float ss[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                U[4 * q4 + j4] *= ss[j4];
                wmx = fmaxf(wmx, fabsf(U[4 * q4 + j4]));
            }
        }
        const int eW = fp16_exp(wave_max(wmx));
        const float scW = ldexpf(1.f, eW);
        const half8 Wf0 = to_frag(U, 0, scW);
        const half8 Wf1 = to_frag(U, 1, scW);
        const float pre = ldexpf(egC, sig + eW);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            floatx16 acc = Sacc[a] * pre;
            acc = mfma32(frag_perm(sm.kct, TST, 32 * a + l32, 0, lane), Wf0, acc);
            acc = mfma32(frag_perm(sm.kct, TST, 32 * a + l32, 16, lane), Wf1, acc);
            Sacc[a] = acc;
        }
        sig = -eW;

        t0 += lc;
        if (ne < ne_end && P.emit_after[ne] == t0) {
            store_state(P.emit_base + (((int64_t)b * P.M + P.emit_slot[ne]) * H + h) * DV * DK, Sacc,
                        sig, w, l32, hi32);
            ++ne;
        }
        lc = lcn;
    }

    store_state(P.state_out + ((int64_t)b * H + h) * DV * DK, Sacc, sig, w, l32, hi32);
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
