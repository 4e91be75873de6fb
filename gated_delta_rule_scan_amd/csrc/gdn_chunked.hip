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
//     (I + A) U = diag(beta) B~,  A_ts = beta_t 2^{g_t - g_s} (k_t . k_s)  (s < t),
//                                 B~_t = v_t - 2^{g_t} S_0 k_t,
// so that, with T = (I + A)^{-1} (it depends on keys and gates only):
//     U   = (T diag(beta)) B~
//     o_t = 2^{g_t} S_0 q_t + sum_{s<=t} 2^{g_t - g_s} (q_t . k_s) u_s
//     S_C = 2^{g_C} S_0 + sum_s 2^{g_C - g_s} u_s k_s^T.
// This is the compact-WY way of applying a product of rank-1 modifications of
// the identity (Golub & Van Loan, Matrix Computations, §5.1) to the chunk.
//
// Key side (state independent, one chunk ahead of the state chain):
//  - all waves convert the next chunk's keys/queries to unit fp16 rows;
//  - T is formed in registers: the Gram tiles come out of MFMA in accumulator
//    layout, and because the Gram matrix is symmetric both A and A^T are
//    available elementwise.  In each 16 x 16 diagonal tile (wave 0: tile 0,
//    wave 2: tile 1) the 8 x 8 diagonal blocks are inverted in the product form
//    (I + N)^{-1} = (I - N)(I + N^2)(I + N^4) (N^8 = 0), then a doubling step
//    X_10 = -X_11 A_10 X_00 gives the tile's inverse; wave 3 forms A_10 of the
//    two tiles and, one barrier later, the last doubling step and the fp16
//    copy.  An MFMA A operand of X is X^T in accumulator layout, so X and X^T
//    are carried side by side where needed;
//  - wave 1 forms P_ts = 2^{g_t - g_s} (q_t . k_s).
// State side (each wave owns 32 value rows): the state is kept transposed
// (S^T, d_k x d_v) in v_mfma_f32_32x32x16_f16 accumulator layout, fp32, as
// S = 2^{-sigma} Sacc.  The decay 2^{g_C} of a chunk is folded into sigma
// rather than applied to Sacc; Sacc is rescaled only when a running bound on
// max|Sacc| leaves the fp16 band.  The accumulator slots feed back as MFMA B
// operands (their reduction index is permuted the same way on both operands).
//
// Operands that the MFMA wants "down a column" (K^T for the state update, V,
// T and P as A operands) are read with ds_read_b64_tr_b16 from token-major LDS
// tiles, so nothing is written transposed.  Keys/queries are stored with the
// middle two 4-column groups of every 16 columns swapped, so that a lane's
// 8-element fragment of the permuted reduction order is one 16-byte read; their
// rows are padded to 272 bytes and permuted (krow) so that every read pattern
// is free of bank conflicts and each lane addresses a tile from one base
// register plus immediate offsets.
//
// Precision: products run on fp16 MFMA with float32 accumulation.  Every fp16
// operand is kept inside the fp16 normal range by exact power-of-two scales
// (checked per chunk; the common case needs none).  The state never leaves
// float32.
//
// Work split: one workgroup of 4 waves per (request, head), two workgroups per
// CU (LDS 80 KB each).  Launches with at most one workgroup per CU use eight
// waves instead: waves 0-3 the state side, waves 4-7 the key side of the same
// schedule, so that the two overlap within each phase.  Inputs go from HBM straight into LDS with
// global_load_lds_dwordx4: raw bf16 key and query rows two chunks ahead of
// the state chain (converted to the fp16 tiles one chunk ahead), V rows one
// chunk ahead; wave 3 issues the key and V copies of the whole workgroup.
// Outputs of a chunk are staged in LDS and stored as whole rows during the
// next one.  Work items without outputs (zero-start replays and transition
// products of the split prefill) run the instantiation without the query side.
//
// Per chunk n, two barriers: after the first, the state chain of n up to B~
// (which needs no T), the conversion of n + 1 and the last step of T for n;
// after the second, the tile tasks of n + 1 and the rest of the state chain
// of n.
#include <atomic>

#include "gdn_launch.h"
#include "gdn_numeric.h"

namespace gdn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef short i16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) void lvoid_t;
typedef __attribute__((address_space(1))) char gchar;  // global memory (so that no flat access is emitted)

constexpr int C = 32;        // tokens per chunk
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int NW = 4;        // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int NVB = 2;       // V staging buffers (copies run one chunk ahead)
constexpr int KS = DK + 8;   // key/query tile row stride (halves)
constexpr int KROWB = 2 * KS;
constexpr int KBUF = C * KROWB;  // bytes of one key/query tile
constexpr float kSigMax = 96.f;  // largest state exponent sigma kept between chunks (S = 2^-sigma Sacc)

struct Smem {
    alignas(16) _Float16 kh[2][C * KS];  // unit keys, fp16 (layout: krow and the column order below)
    alignas(16) _Float16 qh[2][C * KS];  // q' (q as stored, or q / 2^E), fp16 (same layout)
    alignas(16) uint16_t kqr[2][C * DK];  // raw bf16 keys, queries of the chunk after next: [token][column]
    alignas(16) uint16_t vr[NVB][NW][C * 32];  // raw bf16 v: [wave][token][32 value columns]
    alignas(16) _Float16 tT[2][C * C];   // (T diag(beta))^T * 2^eT as fp16 hi [0] + lo [1], row s, column t
    alignas(16) _Float16 pT[2][C * C];   // P^T, row s, column t
    alignas(16) float gl[2][C];          // chunk-local prefix sum of log2 alpha (gl[C-1]: the chunk's total)
    alignas(16) float be[2][C];          // beta (0 past the chunk)
    alignas(16) float eg[2][C];          // 2^{g_t}
    alignas(16) float ws[2][C];          // 2^{g_C - g_t}
    alignas(16) float ks[2][C];          // 1 / ||k'_t||: scale of the stored key row k'_t (0 past the chunk)
    alignas(16) float kq[2][C];          // query scale q = kq q': 1/||q'_t|| (normalised queries) or 2^{E_t}
    alignas(16) float cw[NW][4][C];      // per-wave coefficients (see the state side)
    alignas(16) half8 tpart[2][64];      // T_00, T_11^T tiles (accumulator layout) per lane, fp16 hi (0-3) and lo (4-7)
    int tflag[2];                        // tile b: kTileIll (see key_side_tile_out)
    float tsc;                           // 2^{-eT}
    int tlo;                             // T of the chunk has a lo part (the combine took the hi/lo form)
};
constexpr uint32_t OFF_KH = offsetof(Smem, kh);
constexpr uint32_t OFF_QH = offsetof(Smem, qh);
constexpr uint32_t OFF_VR = offsetof(Smem, vr);
constexpr uint32_t OFF_KQR = offsetof(Smem, kqr);
constexpr uint32_t OFF_TT = offsetof(Smem, tT);
constexpr uint32_t OFF_PT = offsetof(Smem, pT);
constexpr uint32_t OFF_CW = offsetof(Smem, cw);
static_assert(OFF_QH == OFF_KH + 2 * KBUF, "query tiles follow the key tiles");
static_assert(sizeof(Smem) <= 81920, "two workgroups must share a CU's 160 KiB of LDS");

// ---- LDS layouts -------------------------------------------------------------
// Key/query tiles: token t occupies row krow(t) (272 bytes, so row r starts at
// bank 4 (r mod 16) of the 64 four-byte banks).  Actual column c is stored at
// 16 (c/16) + 4 sqd((c/4) % 4) + c % 4 (the middle 4-column groups swapped), in
// 16-byte units u = stored column / 8.  The row order keeps the reads below
// free of bank conflicts: one unit of 32 consecutive rows (16-byte reads, which
// the LDS serves in 16-lane groups), four consecutive tokens x 64 bytes
// (transposed 8-byte reads, served 32 lanes at a time) and 16 rows x units
// 4g + ks, g = lane / 16 (the tile tasks).  Within each half of the tile the
// order is a 4 x 4 transpose, so rows 4 b + j (j = 0..3) of a 4-row block sit
// at 4 j + b % 4 (+16 for b >= 4): one lane term plus a constant per block.
__device__ __forceinline__ int krow(int t) { return 4 * (t & 3) + ((t >> 2) & 3) + (t & 16); }
__device__ __forceinline__ int sqd(int q) { return ((q & 1) << 1) | (q >> 1); }

__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_(float x) { return __builtin_amdgcn_logf(x); }

template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWMASK,
                                                                  0xf, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0x140>(x);  // row_mirror
    return x;
}
// Maxima of non-negative floats as unsigned integers (same order, no NaN
// canonicalisation), one DPP max per step.
__device__ __forceinline__ uint32_t row16_umax(uint32_t x) {
    x = max(x, dppu<0xB1>(x));
    x = max(x, dppu<0x4E>(x));
    x = max(x, dppu<0x141>(x));
    x = max(x, dppu<0x140>(x));
    return x;
}
__device__ __forceinline__ float row16_max(float x) { return __uint_as_float(row16_umax(__float_as_uint(x))); }
__device__ __forceinline__ float lane_val(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// Maximum over the wave of non-negative values (all lanes active), uniform.
__device__ __forceinline__ float wave_max(float x) {
    const uint32_t m = row16_umax(__float_as_uint(x));
    const uint32_t a = __builtin_amdgcn_readlane(m, 0), b = __builtin_amdgcn_readlane(m, 16);
    const uint32_t c = __builtin_amdgcn_readlane(m, 32), d = __builtin_amdgcn_readlane(m, 48);
    return __uint_as_float(max(max(a, b), max(c, d)));
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

// Value held by lane l ^ 32.
__device__ __forceinline__ float partner32(float x, int lane) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(lane < 32 ? r[1] : r[0]);
}
// True when the wave maximum of the per-lane maxima m may leave [2^-6, 2^14)
// (the fp16 band of f16_adjust): some lane at or above 2^14, or all below 2^-6.
__device__ __forceinline__ bool out_of_band(float m) {
    return __builtin_amdgcn_ballot_w64(m >= 0x1p14f) != 0 || __builtin_amdgcn_ballot_w64(m >= 0x1p-6f) == 0;
}

// Power-of-two exponent e for an fp16 operand with maximum magnitude mx: 0 when
// mx is already in [2^-6, 2^14), else the one bringing mx into [2^7, 2^8).
__device__ __forceinline__ int f16_adjust(float mx) {
    if (!(mx > 0.f) || (mx >= 0x1p-6f && mx < 0x1p14f)) return 0;
    int E;
    frexpf(mx, &E);
    // at most 2^120 up (values near the float32 denormal range are
    // negligible next to the state they update), so 2^e stays finite
    return min(8 - E, 120);
}

__device__ __forceinline__ float bf(uint16_t b) { return bf16_to_f32(b); }
__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const float2v f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ half8 cat(half4 a, half4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }

// LDS accesses by byte offset from the workgroup's Smem.
template <typename T>
__device__ __forceinline__ T lds_ld(const Smem &sm, uint32_t off) {
    return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(&sm) + off);
}
template <typename T>
__device__ __forceinline__ void lds_st(Smem &sm, uint32_t off, T v) {
    *reinterpret_cast<T *>(reinterpret_cast<char *>(&sm) + off) = v;
}
// 4 halves of a 16-lane transposed read: lane n of each 16-lane group gets
// element n % 4 of the 8 bytes addressed by lane 4 j + n / 4, for j = 0..3.
__device__ __forceinline__ half4 tr4(const Smem &sm, uint32_t off) {
    const char *p = reinterpret_cast<const char *>(&sm) + off;
    return __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)(p)));
}
__device__ __forceinline__ i16x4_t tr4u(const Smem &sm, uint32_t off) {
    const char *p = reinterpret_cast<const char *>(&sm) + off;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

__device__ __forceinline__ half4 h4(floatx4 x) {
    half4 r;
    r[0] = (_Float16)x[0]; r[1] = (_Float16)x[1]; r[2] = (_Float16)x[2]; r[3] = (_Float16)x[3];
    return r;
}
// Slots 8*hf .. 8*hf+7 of a 32x32 accumulator as an fp16 B fragment.
__device__ __forceinline__ half8 to_frag(const floatx16 &acc, int hf) {
    half8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (_Float16)acc[8 * hf + j];
    return r;
}

__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x16_f16: lane i holds A[i%16][4(i/16)+j] and B[4(i/16)+j][i%16];
// D[4(i/16)+j][i%16] is laid out like B, so the A operand of a matrix X is
// X^T in accumulator layout.
__device__ __forceinline__ floatx4 mm16(half4 a, half4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}
// Lane l copies 16 bytes from base + voff to (LDS base) + 16 l.  Inline
// assembly with an SGPR base, so that the compiler neither waits for it nor
// orders LDS accesses of other buffers behind it.  The copy takes its LDS
// address from m0, which the statement sets; the compiler keeps no value of
// its own in m0 in these kernels (their generated code reads m0 nowhere else),
// so nothing it relies on is overwritten.
__device__ __forceinline__ void dma16(uint64_t base, uint32_t voff, uint32_t lds_wave_base) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_wave_base);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

// ---- per-lane constants ----------------------------------------------------------
struct Lane {
    int lane, l32, hi32, g, n16;
    uint32_t yz;        // Y/Z A fragments: row krow(l32), unit hi32 (+32 bytes per step)
    uint32_t kt[2][2];  // K^T A fragments: [k-step hf][token + 8]
    uint32_t task[2];   // tile-task fragments of rows 16 b + lane%16 (+16 bytes per k-step)
    uint32_t cvt;       // conversion stores of row 4 b + lane/16, block b = 0 (krow)
    uint32_t st;        // transposed reads of T^T / P^T
    uint32_t vrd;       // transposed reads of the wave's V slice
    uint32_t vrdr;      // the same reads from a raw key tile (q = k = v): row stride 256 bytes, wave w at +64 w
    uint32_t cwr;       // this wave's coefficient rows, lane half hi32
    uint32_t ld[2];     // global byte offsets of the key/query rows 8 w + 4 j + lane/16 (copy j)
    uint32_t ldc;       // column part of ld (16 bytes per lane of a row)
    uint32_t vld[2];    // global byte offsets of the V rows 16 k + lane/4
    uint32_t vldc;
    uint32_t gld;       // global byte offset of the gate of token lane%32
    uint32_t ow[4];     // output staging: stores of tokens 8 q4 + 4 hi32 .. +3 of column 32 w + lane%32
    uint32_t orr[2][2]; // output staging: transposed reads [row group k][column half]
    uint32_t ost;       // output store offset: row (lane%16)%4 (+ 8 w + 4 k), columns 32 (lane/16) + 8 ((lane%16)/4) .. +7
};

// Output staging tile of a chunk (32 tokens x 128 value columns, bf16, in the
// chunk's V buffer once every wave's B~ has consumed it): wave w's columns
// 32 w + c hold 8 slots of 4 consecutive tokens each, slot s at byte
// 2048 w + 64 c + 8 (s ^ ostg(c) ^ (w & 1)).  The swizzle keeps the 8-byte
// stores (one slot of 32 columns) and the transposed reads that rebuild full
// token rows (one slot of 16 columns from each of two waves per 32 lanes) free
// of bank conflicts.
__device__ __forceinline__ int ostg(int c) { return (((c >> 3) & 1) << 2) | (((c >> 4) & 1) << 1) | ((c >> 2) & 1); }
__device__ __forceinline__ uint32_t ostage(int w, int c, int slot) {
    return 2048 * w + 64 * c + 8 * (slot ^ ostg(c) ^ (w & 1));
}

__device__ __forceinline__ Lane make_lane(int tid, int w, int H) {
    Lane L;
    L.lane = tid & 63;
    L.l32 = L.lane & 31;
    L.hi32 = L.lane >> 5;
    L.g = L.lane >> 4;
    L.n16 = L.lane & 15;
    const int g = L.g, n = L.n16;
    L.yz = krow(L.l32) * KROWB + 16 * L.hi32;
    {
        const int s = sqd(n & 3);
        const uint32_t col = (2 * (g & 1) + (s >> 1)) * 16 + 8 * (s & 1);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int d8 = 0; d8 < 2; ++d8)
                L.kt[hf][d8] = krow(16 * hf + 4 * (g >> 1) + (n >> 2) + 8 * d8) * KROWB + col;
    }
    L.task[0] = krow(n) * KROWB + 64 * g;
    L.task[1] = krow(16 + n) * KROWB + 64 * g;
    L.cvt = krow(g) * KROWB + 32 * (n >> 1) + 8 * (n & 1);
    L.st = 64 * (4 * (g >> 1) + (n >> 2)) + 2 * (16 * (g & 1) + 4 * (n & 3));
    L.vrd = 64 * (4 * (g >> 1) + (n >> 2)) + 32 * (g & 1) + 8 * (n & 3);
    L.vrdr = 256 * (4 * (g >> 1) + (n >> 2)) + 64 * w + 32 * (g & 1) + 8 * (n & 3);
    L.cwr = OFF_CW + w * 4 * C * 4 + 16 * L.hi32;
    const uint32_t hdk2 = (uint32_t)(H * DK * 2);
    L.ldc = 16 * n;
#pragma unroll
    for (int j = 0; j < 2; ++j) L.ld[j] = (uint32_t)(8 * w + 4 * j + g) * hdk2 + L.ldc;
    L.vldc = 16 * (L.lane & 3);
#pragma unroll
    for (int k = 0; k < 2; ++k) L.vld[k] = (uint32_t)(16 * k + (L.lane >> 2)) * hdk2 + L.vldc;
    L.gld = (uint32_t)(L.l32 * H * 2);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) L.ow[q4] = ostage(w, L.l32, 2 * q4 + L.hi32);
    // transposed read (k, hh) of the rows 8 w + 4 k .. +3 (slot 2 w + k): lane (g, n) supplies the
    // slot of column 8 (n%4) + n/4 + 4 hh of wave g's part, so that it receives token
    // 8 w + 4 k + n%4, columns 32 g + 8 (n/4) + 4 hh .. +3
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) L.orr[k][hh] = ostage(g, 8 * (n & 3) + (n >> 2) + 4 * hh, 2 * w + k);
    L.ost = (uint32_t)(n & 3) * hdk2 + 64 * g + 16 * (n >> 2);
    return L;
}

// ---- chunk schedule ------------------------------------------------------------
struct Chunk {
    int t0, lc, ne;  // first position, length (0: none), first emission not yet taken
};
__device__ __forceinline__ int chunk_len(const LaunchDesc &P, int len, int t0, int e, int e_end) {
    int lc = min(C, len - t0);
    if (e < e_end) lc = min(lc, P.emit_after[e] - t0);
    return lc;
}
__device__ __forceinline__ Chunk next_chunk(const LaunchDesc &P, const Chunk &c, int len, int ne_end) {
    Chunk n;
    n.t0 = c.t0 + c.lc;
    n.ne = c.ne;
    if (n.ne < ne_end && P.emit_after[n.ne] == n.t0) ++n.ne;
    n.lc = (c.lc > 0 && n.t0 < len) ? chunk_len(P, len, n.t0, n.ne, ne_end) : 0;
    return n;
}

// ---- loads ---------------------------------------------------------------------
struct Pref {
    uint16_t ga, gb;   // wave 1: alpha, beta of token lane%32
};

// Byte addresses of the span's first token (head h) in each packed tensor and
// the byte strides between consecutive tokens; a chunk starting at span token
// t0 is at base + t0 * stride.
struct Bases {
    uint64_t k, q, v, a, b, o;  // v: the wave's 32 value columns
    uint32_t ts;                // H d * 2 (rows of q, k, v, o; d_k = d_v = d)
    uint32_t tg;                // H * 2 (alpha, beta)
};
__device__ __forceinline__ uint64_t at_tok(uint64_t base, int t0, uint32_t stride) {
    return base + (uint64_t)(uint32_t)t0 * stride;
}

// Keys (and queries) of a chunk into the raw tiles: wave w copies rows
// 8 w .. 8 w + 7, 1 KiB (4 rows) per copy, lane l taking row 8 w + 4 j + l/16,
// columns 8 (l%16) .. +7.  Rows past the chunk are clamped to its last row
// (always in the span), so that every copy is issued; their values are ignored
// by the consumers.  The gates (wave 1) go to registers.  t0 is the chunk's
// first span token.
// WHICH = 0: keys; 1: queries (when COPY) and, from wave 1, the gates.
template <int WHICH, bool COPY = true>
__device__ __forceinline__ void load_kq(Pref &pf, uint32_t sm_lds, const Bases &G, int t0, int lc, int w,
                                        const Lane &L, uint32_t tile = OFF_KQR + WHICH * C * DK * 2) {
    const uint64_t base = at_tok(WHICH ? G.q : G.k, t0, G.ts);
    const uint32_t lim = (uint32_t)(lc - 1) * G.ts + L.ldc;
    if (COPY) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            dma16(base, min(L.ld[j], lim), sm_lds + tile + (uint32_t)((8 * w + 4 * j) * DK * 2));
    }
    if (WHICH == 1 && w == 1) {
        typedef __attribute__((address_space(1))) const uint16_t gu16;
        const gchar *ab = (const gchar *)at_tok(G.a, t0, G.tg);
        const gchar *bb = (const gchar *)at_tok(G.b, t0, G.tg);
        const uint32_t off = min(L.gld, (uint32_t)(lc - 1) * G.tg);
        pf.ga = *(gu16 *)(ab + off);
        pf.gb = *(gu16 *)(bb + off);
    }
}

// V rows of a chunk into the wave's slice of buffer vb: copy k covers rows
// 16 k .. 16 k + 15, lane l taking row 16 k + l/4, value columns
// 32 w + 8 (l%4) .. +7 (LDS: slice + 1 KiB k + 16 l).
// sm_lds is the LDS byte address of the workgroup's Smem.
__device__ __forceinline__ void dma_v(uint32_t sm_lds, int vb, const Bases &G, int t0, int lc, int w,
                                      const Lane &L) {
    const uint64_t base = at_tok(G.v, t0, G.ts);
    const uint32_t lim = (uint32_t)(lc - 1) * G.ts + L.vldc;
#pragma unroll
    for (int k = 0; k < 2; ++k)
        dma16(base, min(L.vld[k], lim), sm_lds + OFF_VR + (uint32_t)(((vb * NW + w) * C * 32 + 16 * k * 32) * 2));
}

// Wave 3 copies the key rows and the V columns of all four waves (the other
// waves carry the longer tile tasks in the same phase).
__device__ __forceinline__ void load_k_all(uint32_t sm_lds, const Bases &G, int t0, int lc, const Lane &L,
                                           uint32_t tile = OFF_KQR) {
    const uint64_t base = at_tok(G.k, t0, G.ts);
    const uint32_t lim = (uint32_t)(lc - 1) * G.ts + L.ldc;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            dma16(base, min(L.ld[j] - (uint32_t)(8 * (3 - w2)) * G.ts, lim),
                  sm_lds + tile + (uint32_t)((8 * w2 + 4 * j) * DK * 2));
}
__device__ __forceinline__ void dma_v_all(uint32_t sm_lds, int vb, const Bases &G, int t0, int lc, const Lane &L) {
    const uint64_t base3 = at_tok(G.v, t0, G.ts);  // G.v holds wave 3's columns
    const uint32_t lim = (uint32_t)(lc - 1) * G.ts + L.vldc;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2)
#pragma unroll
        for (int k = 0; k < 2; ++k)
            dma16(base3 - (uint64_t)(64 * (3 - w2)), min(L.vld[k], lim),
                  sm_lds + OFF_VR + (uint32_t)(((vb * NW + w2) * C * 32 + 16 * k * 32) * 2));
}

// ---- key side, part 1 (all waves): fp16 keys / queries and gate sums -------------
// Keys are kept as stored: a bf16 row is exact in fp16 (8 significant bits)
// when its elements lie in the fp16 range, and the normalisation 1/||k|| goes
// into per-token coefficients (ks) instead of being rounded into the row.
// A lane converts the 8 columns of one row (16-byte unit pair).  The
// conversion of a wave's rows is split in three steps so that the rows'
// latency chains overlap: row_load (unpack, squared norm), the general form
// for the 4-row blocks that need it (row_general, rare), row_store (fp16 store
// at LDS byte offset dst, the upper unit at +16; returns the row's scale s
// with k^ = s k', k' the stored fp16 row, 0 for rows past the chunk).
struct RowCv {
    float f[8];
    float ss;  // squared norm of the row (all 16 lanes of the row)
};
__device__ __forceinline__ void row_load(RowCv &r, uint4 raw) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r.f[2 * e] = bflo(wd[e]);
        r.f[2 * e + 1] = bfhi(wd[e]);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16x2v pr = __builtin_bit_cast(bf16x2v, wd[e]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
    }
    r.ss = row16_sum(ss);  // one token row per 16 lanes
}
// A row with ||k|| in [1/2, 2) is stored as it is (unit keys always are).
// Any other row sends its 4-row block through the general form: each row is
// scaled by the power of two that brings its largest element into [1/2, 1)
// (exact), so that it fits fp16 and its squared norm lies in [1/4, d_k]; this
// also covers squared norms that overflow or underflow float32.  A zero row
// keeps scale 0 (it stays zero).
__device__ __forceinline__ bool row_needs_general(const RowCv &r, bool live) {
    return live && !(r.ss >= 0.25f && r.ss < 4.f);
}
__device__ __forceinline__ void row_general(RowCv &r) {
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(r.f[e]));
    mx = row16_max(mx);
    const int E = __builtin_amdgcn_frexp_expf(mx);  // mx = m 2^E, m in [1/2, 1)
    float s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        r.f[e] = __builtin_amdgcn_ldexpf(r.f[e], -E);
        s2 = fmaf(r.f[e], r.f[e], s2);
    }
    r.ss = row16_sum(s2);
}
__device__ __forceinline__ float row_store(Smem &sm, uint32_t dst, const RowCv &r, bool live) {
    half4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = (_Float16)r.f[e];
        hi[e] = (_Float16)r.f[4 + e];
    }
    lds_st(sm, dst, lo);
    lds_st(sm, dst + 16, hi);
    return (live && r.ss > 0.f) ? __builtin_amdgcn_rsqf(r.ss) : 0.f;
}
// The same conversion for one row, in one piece (fewer live registers; the
// four-wave kernel converts row by row).  Same results as the three steps.
__device__ __forceinline__ float convert_key_row(Smem &sm, uint32_t dst, uint4 raw, bool live) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = bflo(wd[e]);
        f[2 * e + 1] = bfhi(wd[e]);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16x2v pr = __builtin_bit_cast(bf16x2v, wd[e]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
    }
    ss = row16_sum(ss);  // one token row per 16 lanes
    float s = live ? __builtin_amdgcn_rsqf(ss) : 0.f;
    // A row with ||k|| in [1/2, 2) is stored as it is (unit keys always are).
    // Any other row sends the wave through the general form: the row is scaled
    // by the power of two that brings its largest element into [1/2, 1)
    // (exact), so that it fits fp16 and its squared norm lies in [1/4, d_k];
    // this also covers squared norms that overflow or underflow float32.  A
    // zero row keeps scale 0 (it stays zero).
    if (__builtin_amdgcn_ballot_w64(live && !(ss >= 0.25f && ss < 4.f)) != 0) {
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(f[e]));
        mx = row16_max(mx);
        const int E = __builtin_amdgcn_frexp_expf(mx);  // mx = m 2^E, m in [1/2, 1)
        float s2 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            f[e] = __builtin_amdgcn_ldexpf(f[e], -E);
            s2 = fmaf(f[e], f[e], s2);
        }
        s2 = row16_sum(s2);
        s = (live && s2 > 0.f) ? __builtin_amdgcn_rsqf(s2) : 0.f;
    }
    half4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = (_Float16)f[e];
        hi[e] = (_Float16)f[4 + e];
    }
    lds_st(sm, dst, lo);
    lds_st(sm, dst + 16, hi);
    return s;
}

// Queries used as stored (no GDN_NORMALIZE_Q): converts the 8 columns of one
// lane scaled by the power of two 2^-E that brings the row's largest element
// into [1/2, 1) (exact), with 2^E returned in kq_out; stored like row_store.
// (Normalised queries take the key steps: they are kept as stored too, their
// 1/||q|| going into per-token coefficients.)
__device__ __forceinline__ void convert_query_row_scaled(Smem &sm, uint32_t dst, uint4 raw, bool live,
                                                         float *kq_out) {
    // rows past the chunk hold a copy of a live row (finite); they get scale 0
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = bflo(wd[e]);
        f[2 * e + 1] = bfhi(wd[e]);
    }
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(f[e]));
    mx = row16_max(mx);
    int E = 0;
    frexpf(mx, &E);
    const float sc = live ? ldexpf(1.f, -E) : 0.f;
    *kq_out = ldexpf(1.f, E);
    half4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = (_Float16)(f[e] * sc);
        hi[e] = (_Float16)(f[4 + e] * sc);
    }
    // actual 4-column groups 2(u%2), 2(u%2)+1 of 16-group u/2 -> stored groups u%2, 2 + u%2
    lds_st(sm, dst, lo);
    lds_st(sm, dst + 16, hi);
}

// Conversion work of a chunk in 4-row blocks: block b of the keys (and, with
// outputs, of the queries) covers tokens 4 b .. 4 b + 3, lane l converting
// token 4 b + l/16, columns 8 (l%16) .. +7.  With outputs, waves 0 and 2 take
// five blocks each, wave 1 (which also forms the gate sums) four and wave 3
// (which also finishes T in this phase) two; keys alone go three to waves 0
// and 2 each, two to wave 1 and none to wave 3.
// With eight key-side waves (NK = 8, the d_v-split kernel) roles 0 and 2
// convert three blocks each, roles 1 and 3-6 two (role 1 also forms the gate
// sums) and role 7, which finishes T in the same phase, none.
template <bool WANT_Q, int NK = 4>
__device__ constexpr int cvt_owner(int gi) {  // gi: block gi/2 of keys (gi even) or queries
    if (NK == 8) {
        const int kind = WANT_Q ? (gi & 1) : 0, rb = WANT_Q ? (gi >> 1) : gi;
        return kind == 0 ? (rb < 2 ? 0 : rb < 4 ? 2 : rb - 1)
                         : (rb < 2 ? 1 : rb == 2 ? 3 : rb == 3 ? 4 : rb == 4 ? 0 : rb == 5 ? 5 : rb == 6 ? 2 : 6);
    }
    return WANT_Q ? (gi < 5 ? 0 : gi < 10 ? 2 : gi < 14 ? 1 : 3) : (gi < 3 ? 0 : gi < 5 ? 1 : 2);
}


// BATCH: the norms of all of the wave's rows before any store (waves that do
// only key-side work); otherwise row by row (fewer live registers).  Both
// give the same results.
template <bool WANT_Q, bool NORM_Q, int W, int NK = 4, bool BATCH = false>
__device__ __forceinline__ void key_side_convert(Smem &sm, int pb, const Pref &pf, int lc, const Lane &L,
                                                 uint32_t rawk = OFF_KQR, uint32_t rawq = OFF_KQR + C * DK * 2) {
    const uint32_t kbuf = OFF_KH + pb * KBUF, qbuf = OFF_QH + pb * KBUF;
    constexpr int NG = WANT_Q ? 16 : 8;
    // all raw rows of this wave are read before the first converted row is
    // stored, so that the reads overlap instead of each waiting behind a store
    uint4 raw[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        if (cvt_owner<WANT_Q, NK>(gi) != W) continue;
        const int kind = WANT_Q ? (gi & 1) : 0;
        const int rb = WANT_Q ? (gi >> 1) : gi;
        raw[gi] = lds_ld<uint4>(sm, (kind ? rawq : rawk) + (uint32_t)(rb * 4 * DK * 2) + 16 * L.lane);
    }
    // keys and normalised queries: a row's norm, the rare general form per
    // 4-row block, the store; with BATCH the norms of all of the wave's rows
    // come first, so that their latency chains overlap
    constexpr bool QN = WANT_Q && NORM_Q;
    RowCv rc[NG];
    bool gen[NG];
    auto load_block = [&](int gi) {
        const int rb = WANT_Q ? (gi >> 1) : gi;
        row_load(rc[gi], raw[gi]);
        gen[gi] = row_needs_general(rc[gi], 4 * rb + L.g < lc);
    };
    auto store_block = [&](int gi) {
        const int kind = WANT_Q ? (gi & 1) : 0;
        const int rb = WANT_Q ? (gi >> 1) : gi;
        const int t = 4 * rb + L.g;
        const bool live = t < lc;
        const uint32_t dst = (kind ? qbuf : kbuf) + L.cvt + (uint32_t)(((rb & 3) + 16 * (rb >> 2)) * KROWB);
        if (kind == 0) {
            const float ksv = row_store(sm, dst, rc[gi], live);
            if (L.n16 == 0) sm.ks[pb][t] = ksv;
        } else {
            // kq: 1/||q'|| of a normalised query, or the power of two of a query used as stored
            float kqv;
            if (NORM_Q) kqv = row_store(sm, dst, rc[gi], live);
            else convert_query_row_scaled(sm, dst, raw[gi], live, &kqv);
            if (L.n16 == 0) sm.kq[pb][t] = kqv;
        }
    };
    if (BATCH) {
        bool any = false;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            if (cvt_owner<WANT_Q, NK>(gi) != W || (WANT_Q && (gi & 1) && !QN)) continue;
            load_block(gi);
            any = any || gen[gi];
        }
        if (__builtin_amdgcn_ballot_w64(any) != 0) {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                if (cvt_owner<WANT_Q, NK>(gi) != W || (WANT_Q && (gi & 1) && !QN)) continue;
                if (__builtin_amdgcn_ballot_w64(gen[gi]) != 0) row_general(rc[gi]);
            }
        }
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            if (cvt_owner<WANT_Q, NK>(gi) != W) continue;
            store_block(gi);
        }
    } else {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            if (cvt_owner<WANT_Q, NK>(gi) != W) continue;
            const int kind = WANT_Q ? (gi & 1) : 0;
            const int rb = WANT_Q ? (gi >> 1) : gi;
            const int t = 4 * rb + L.g;
            const bool live = t < lc;
            const uint32_t dst = (kind ? qbuf : kbuf) + L.cvt + (uint32_t)(((rb & 3) + 16 * (rb >> 2)) * KROWB);
            if (kind == 0) {
                const float ksv = convert_key_row(sm, dst, raw[gi], live);
                if (L.n16 == 0) sm.ks[pb][t] = ksv;
            } else {
                float kqv;
                if (NORM_Q) kqv = convert_key_row(sm, dst, raw[gi], live);
                else convert_query_row_scaled(sm, dst, raw[gi], live, &kqv);
                if (L.n16 == 0) sm.kq[pb][t] = kqv;
            }
        }
    }
    constexpr int w = W;
    if (w == 1) {
        const int tl = L.l32;
        const bool live = tl < lc;
        const float av = bf(pf.ga);
        const float lg = live ? log2_(fmaxf(av, 1e-30f)) : 0.f;
        const float gs = scan32(lg);
        const float gC = lane_val(gs, C - 1);
        if (L.lane < 32) {
            sm.gl[pb][tl] = gs;
            sm.eg[pb][tl] = exp2_(gs);
            sm.ws[pb][tl] = exp2_(gC - gs);
        } else {
            sm.be[pb][tl] = live ? bf(pf.gb) : 0.f;
        }
    }
}

// Raw key (and query) rows of the 4-token blocks that wave W converts (the
// owner map of key_side_convert), for the chunk at span token t0 with lc rows;
// rows past the chunk are clamped to its last row.  A wave that copies exactly
// the rows it converts may issue the copies right after its own conversion.
template <bool WANT_Q, int W, int NK = 4>
__device__ __forceinline__ void load_owned(uint32_t sm_lds, const Bases &G, int t0, int lc, const Lane &L) {
    const uint32_t lim = (uint32_t)(lc - 1) * G.ts + L.ldc;
    constexpr int NG = WANT_Q ? 16 : 8;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        if (cvt_owner<WANT_Q, NK>(gi) != W) continue;
        const int kind = WANT_Q ? (gi & 1) : 0;
        const int rb = WANT_Q ? (gi >> 1) : gi;
        dma16(at_tok(kind ? G.q : G.k, t0, G.ts), min((uint32_t)(4 * rb + L.g) * G.ts + L.ldc, lim),
              sm_lds + OFF_KQR + (uint32_t)(kind * C * DK * 2 + rb * 4 * DK * 2));
    }
}

// ---- key side, part 2: T = (I + A)^{-1} in three tile tasks and a combine ----
// Tile-task operand fragments: rows 16 b + lane%16, k-step ks covering the
// 16-byte units 4 (lane/16) + ks (the same units on both MFMA operands).
__device__ __forceinline__ void task_frags(const Smem &sm, uint32_t buf, uint32_t base, half8 (&f)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) f[ks] = lds_ld<half8>(sm, buf + base + 16 * ks);
}

// fp16 hi/lo pair of float32 values: x = hi + lo to about 2^-22 relative.
__device__ __forceinline__ void split16(const floatx4 &x, half4 &hi, half4 &lo) {
    hi = h4(x);
    floatx4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = x[j] - (float)hi[j];
    lo = h4(r);
}
__device__ __forceinline__ floatx4 f4(half4 x) {
    floatx4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (float)x[j];
    return r;
}

// Diagonal tile b (tokens 16b .. 16b+15), wave 0 (b = 0) or wave 2 (b = 1):
// T_bb, returned for b = 0 as T_00 and for b = 1 as T_11^T (both in
// accumulator layout: lane i holds rows 4(i/16) + j, column i%16).
//
// The product form gives a first inverse T0 = R - R L R (R the 8 x 8
// block-diagonal inverse, L the lower-left block); its fp16 intermediates lose
// accuracy when the keys of the tile are nearly parallel and beta approaches
// 2 (entries of N^2, N^4 far above those of the inverse).  For a tile with an
// entry |A_ts| >= kIll (`ill`, uniform over the wave) one Newton step,
//     T1 = T0 + T0 E,   E = I - (I + A) T0,
// with A (float32) applied as an fp16 hi/lo pair and T0 exact in fp16,
// squares the relative error of T0.  Below kIll the fp16 product form is
// already within about 1.3e-4 (relative Frobenius) of the exact inverse, less
// than one fp16 rounding of T, so the step is skipped.
constexpr float kIll = 0.5f;
__device__ __forceinline__ floatx4 key_side_tile(const Smem &sm, int pb, int b, const Lane &L, bool &ill) {
    const int c = L.n16, rb = 4 * L.g;
    half8 f[4];
    task_frags(sm, OFF_KH + pb * KBUF, b ? L.task[1] : L.task[0], f);
    const floatx4 z = {0.f, 0.f, 0.f, 0.f};
    floatx4 G = z;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) G = mfma16(f[ks], f[ks], G);
    const float *gl = sm.gl[pb];
    const float *be = sm.be[pb];
    const float *kn = sm.ks[pb];
    half4 id4;
    floatx4 idf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        id4[j] = (_Float16)(rb + j == c ? 1.f : 0.f);
        idf[j] = rb + j == c ? 1.f : 0.f;
    }
    // A (rows > cols) and A^T (rows < cols) of the tile, split into the two
    // 8 x 8 diagonal blocks (N) and the lower-left block (L); the stored keys
    // k' carry their scales ks (k^ = ks k')
    const float gls = gl[16 * b + c], bes = be[16 * b + c], kss = kn[16 * b + c];
    const float4 glt = *reinterpret_cast<const float4 *>(&gl[16 * b + rb]);
    const float4 bet = *reinterpret_cast<const float4 *>(&be[16 * b + rb]);
    const float4 knt = *reinterpret_cast<const float4 *>(&kn[16 * b + rb]);
    const float glv[4] = {glt.x, glt.y, glt.z, glt.w}, bev[4] = {bet.x, bet.y, bet.z, bet.w};
    const float knv[4] = {knt.x, knt.y, knt.z, knt.w};
    floatx4 N, Nt, Lw, Lt;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = rb + j;
        const bool lower = r > c, upper = r < c, same8 = ((r ^ c) & 8) == 0;
        const float d = glv[j] - gls;
        // computed on every lane (the diagonal is dropped by the selects), so
        // that no branch splits the task
        const float val = (lower ? bev[j] : bes) * exp2_(lower ? d : -d) * (knv[j] * kss) * G[j];
        N[j] = (lower && same8) ? val : 0.f;
        Nt[j] = (upper && same8) ? val : 0.f;
        Lw[j] = (lower && !same8) ? val : 0.f;
        Lt[j] = (upper && !same8) ? val : 0.f;
    }
    {
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) am = fmaxf(am, fmaxf(fabsf(N[j]), fabsf(Lw[j])));
        ill = __builtin_amdgcn_ballot_w64(am >= kIll) != 0;
    }
    const half4 Nh = h4(N), Nth = h4(Nt), Lh = h4(Lw), Lth = h4(Lt);
    const floatx4 N2 = mm16(Nth, Nh, z);     // N N
    const floatx4 N2t = mm16(Nh, Nth, z);    // N^T N^T
    const half4 N2h = h4(N2), N2th = h4(N2t);
    const floatx4 N4t = mm16(N2h, N2th, z);  // (N^2)^T (N^2)^T
    const floatx4 N4 = mm16(N2th, N2h, z);   // N^2 N^2
    const floatx4 R1 = mm16(id4 - Nth, id4 + N2h, z);   // (I - N)(I + N^2)
    const floatx4 R1t = mm16(id4 - Nh, id4 + N2th, z);  // (I - N^T)(I + (N^2)^T)
    const floatx4 R = mm16(id4 + h4(N4t), h4(R1), z);   // (I + N^4) R1 = blockdiag inverse
    const floatx4 Rt = mm16(id4 + h4(N4), h4(R1t), z);  // its transpose
    // T0 and T0^T (accumulator layout), R - R L R; the copy not returned is
    // formed only for the Newton step
    floatx4 T0, T0t;
    if (b == 0) {
        const half4 X = h4(mm16(Lth, h4(R), z));  // L R
        T0 = mm16(h4(Rt), -X, R);
        if (!ill) return T0;
        T0t = mm16(X, -h4(Rt), Rt);
    } else {
        const half4 Xt = h4(mm16(Lh, h4(Rt), z));  // (R L)^T
        T0t = mm16(h4(R), -Xt, Rt);
        if (!ill) return T0t;
        T0 = mm16(Xt, -h4(R), R);
    }
    const half4 T0h = h4(T0), T0th = h4(T0t);
    // The two copies of T0 come from separate chains (their roundings
    // differ), so the residual is taken against the copy the step starts
    // from; the error of T1 is then the product of the two copies' errors.
    half4 Ah, Al;
    if (b == 0) {
        // T1 = T0 + T0' E, E = I - T0 - A T0 (A = A_hi + A_lo; the A operand of A T0 is A^T)
        split16(Nt + Lt, Ah, Al);
        floatx4 AT = mm16(Ah, T0h, z);
        AT = mm16(Al, T0h, AT);
        const half4 Eh = h4(idf - f4(T0h) - AT);
        return mm16(T0th, Eh, f4(T0h));
    }
    // T1^T = T0^T + T0'^T E^T, E^T = I - T0^T - A^T T0^T (the left residual I - T0 (I + A), transposed)
    split16(N + Lw, Ah, Al);
    floatx4 AT = mm16(Ah, T0th, z);
    AT = mm16(Al, T0th, AT);
    const half4 Eh = h4(idf - f4(T0th) - AT);
    return mm16(T0h, Eh, f4(T0th));
}

// Wave 3: A_10^T (accumulator layout) from the (0, 1) Gram tile.
__device__ __forceinline__ floatx4 key_side_a10t(const Smem &sm, int pb, const Lane &L) {
    const int c = L.n16, rb = 4 * L.g;
    half8 f0[4], f1[4];
    task_frags(sm, OFF_KH + pb * KBUF, L.task[0], f0);
    task_frags(sm, OFF_KH + pb * KBUF, L.task[1], f1);
    floatx4 G01 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) G01 = mfma16(f0[ks], f1[ks], G01);  // (k_r . k_{16+c})
    const float *gl = sm.gl[pb];
    const float gt = gl[16 + c], bt = sm.be[pb][16 + c] * sm.ks[pb][16 + c];
    const float4 gs4 = *reinterpret_cast<const float4 *>(&gl[rb]);
    const float4 ks4 = *reinterpret_cast<const float4 *>(&sm.ks[pb][rb]);
    const float gsv[4] = {gs4.x, gs4.y, gs4.z, gs4.w}, ksv[4] = {ks4.x, ks4.y, ks4.z, ks4.w};
    floatx4 A10t;
#pragma unroll
    for (int j = 0; j < 4; ++j) A10t[j] = bt * exp2_(gt - gsv[j]) * ksv[j] * G01[j];
    return A10t;
}

// Stores a 4-element part of T diag(beta) (accumulator layout) as its fp16
// hi/lo pair: block 0 = T_00 (rows t = rb + j, column s = c), 1 = T_10
// (t = 16 + rb + j, s = c), 2 = T_11 held transposed (t = 16 + c, s = 16 + rb + j).
// Stored as (row s, column t).
// split = false stores x rounded once, with a zero lo part.
__device__ __forceinline__ void store_tpart(Smem &sm, int blk, const floatx4 &x, int c, int rb, bool split = true) {
    half4 hi, lo = {0, 0, 0, 0};
    if (split) split16(x, hi, lo);
    else hi = h4(x);
    // without the split the lo part is not read (the combine's flag in LDS)
#pragma unroll
    for (int part = 0; part < (split ? 2 : 1); ++part) {
        _Float16 *tt = sm.tT[part];
        const half4 v = part ? lo : hi;
        if (blk == 0) {
            *reinterpret_cast<half4 *>(&tt[c * C + rb]) = v;
        } else if (blk == 1) {
            *reinterpret_cast<half4 *>(&tt[c * C + 16 + rb]) = v;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) tt[(16 + rb + j) * C + 16 + c] = v[j];
        }
    }
}

// Flag of a diagonal tile for the combine (LDS tflag): the tile took the
// Newton step (an |A_ts| >= kIll), so its staged copy carries a lo part.
constexpr int kTileIll = 4;

// Diagonal tile b (wave 0: b = 0, wave 2: b = 1) after key_side_tile: stages
// the tile for the combine, fp16 hi and (when ill) lo.  The tile's block of
// T diag(beta) is written by the combine, in the next phase: the state side
// still reads the current chunk's T during this one.
__device__ __forceinline__ void key_side_tile_out(Smem &sm, int b, const floatx4 &r, bool ill, const Lane &L) {
    half4 hi, lo = {0, 0, 0, 0};
    if (ill) split16(r, hi, lo);
    else hi = h4(r);
    sm.tpart[b][L.lane] = cat(hi, lo);
    if (L.lane == 0) sm.tflag[b] = ill ? kTileIll : 0;
}

// Combine (one wave): T_10 = -T_11 A_10 T_00, then T diag(beta) scaled into
// the fp16 band and stored (row s, column t) as an fp16 hi/lo pair.  When a
// tile took the Newton step or A_10 has an entry >= kIll, both products take
// their operands as hi/lo pairs (three MFMAs each: hi hi, lo hi, hi lo) and T
// keeps float32 accuracy up to the state update; otherwise single fp16
// products and a single fp16 T (zero lo part) are exact to one rounding of T.
// A10t: A_10^T of the chunk, kept in this wave's registers since its task.
__device__ __forceinline__ void key_side_combine(Smem &sm, int pb, const Lane &L, const floatx4 &A10t) {
    const int lane = L.lane;
    const half8 p0 = sm.tpart[0][lane], p1 = sm.tpart[1][lane];
    const int f0 = sm.tflag[0], f1 = sm.tflag[1];
    const half4 th = __builtin_shufflevector(p0, p0, 0, 1, 2, 3), tl = __builtin_shufflevector(p0, p0, 4, 5, 6, 7);
    const half4 uh = __builtin_shufflevector(p1, p1, 0, 1, 2, 3), ul = __builtin_shufflevector(p1, p1, 4, 5, 6, 7);
    const floatx4 z = {0.f, 0.f, 0.f, 0.f};
    float am = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) am = fmaxf(am, fabsf(A10t[j]));
    const bool ill = ((f0 | f1) & kTileIll) != 0 || __builtin_amdgcn_ballot_w64(am >= kIll) != 0;
    floatx4 T10;
    if (ill) {
        half4 ah, al;
        split16(A10t, ah, al);
        floatx4 W = mm16(ah, th, z);  // A_10 T_00 (a tile without the step has lo = 0)
        W = mm16(al, th, W);
        W = mm16(ah, tl, W);
        half4 wh, wl;
        split16(-W, wh, wl);
        T10 = mm16(uh, wh, z);  // -T_11 (A_10 T_00)
        T10 = mm16(ul, wh, T10);
        T10 = mm16(uh, wl, T10);
    } else {
        const floatx4 W = mm16(h4(A10t), th, z);
        T10 = mm16(uh, -h4(W), z);
    }
    const int c = L.n16, rb = 4 * L.g;
    const float bs0 = sm.be[pb][c];  // column s = c (T_00, T_10)
    const float4 b14 = *reinterpret_cast<const float4 *>(&sm.be[pb][16 + rb]);  // columns s = 16 + rb + j (T_11^T)
    const float b1v[4] = {b14.x, b14.y, b14.z, b14.w};
    floatx4 t00, t10, t11;
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        t00[j] = ((float)th[j] + (float)tl[j]) * bs0;
        t10[j] = T10[j] * bs0;
        t11[j] = ((float)uh[j] + (float)ul[j]) * b1v[j];
        mx = fmaxf(mx, fmaxf(fabsf(t00[j]), fmaxf(fabsf(t10[j]), fabsf(t11[j]))));
    }
    const int eT = out_of_band(mx) ? f16_adjust(wave_max(mx)) : 0;
    if (eT != 0) {
        const float sc = ldexpf(1.f, eT);
        t00 *= sc;
        t10 *= sc;
        t11 *= sc;
    }
    store_tpart(sm, 0, t00, c, rb, ill);
    store_tpart(sm, 1, t10, c, rb, ill);
    store_tpart(sm, 2, t11, c, rb, ill);
    if (lane == 0) {
        sm.tsc = ldexpf(1.f, -eT);
        sm.tlo = ill ? 1 : 0;
    }
}

// ---- key side, part 3 (wave 1): P -> fp16, transposed -------------------------
// NORM_Q: the queries' scales 1/||q'|| go into the rows of P (queries used as
// stored keep theirs in the output coefficients instead, where a large scale
// cannot overflow fp16).  QFROMK: the query tile is the key tile (q = k).
template <bool NORM_Q, bool QFROMK>
__device__ __forceinline__ void key_side_P(Smem &sm, int pb, const Lane &L) {
    const int c = L.n16, rb = 4 * L.g;
    half8 k0[4], k1[4], q0[4], q1[4];
    task_frags(sm, OFF_KH + pb * KBUF, L.task[0], k0);
    task_frags(sm, OFF_KH + pb * KBUF, L.task[1], k1);
    task_frags(sm, (QFROMK ? OFF_KH : OFF_QH) + pb * KBUF, L.task[0], q0);
    task_frags(sm, (QFROMK ? OFF_KH : OFF_QH) + pb * KBUF, L.task[1], q1);
    const floatx4 z = {0.f, 0.f, 0.f, 0.f};
    floatx4 P00 = z, P10 = z, P11 = z;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        P00 = mfma16(q0[ks], k0[ks], P00);
        P10 = mfma16(q1[ks], k0[ks], P10);
        P11 = mfma16(q1[ks], k1[ks], P11);
    }
    const float *gl = sm.gl[pb];
    const float g0 = gl[c], g1 = gl[16 + c];
    const float ks0 = sm.ks[pb][c], ks1 = sm.ks[pb][16 + c];  // scales of the stored keys s = c, 16 + c
    const float4 a4 = *reinterpret_cast<const float4 *>(&gl[rb]);
    const float4 b4 = *reinterpret_cast<const float4 *>(&gl[16 + rb]);
    const float gt0[4] = {a4.x, a4.y, a4.z, a4.w}, gt1[4] = {b4.x, b4.y, b4.z, b4.w};
    float qs0[4] = {1.f, 1.f, 1.f, 1.f}, qs1[4] = {1.f, 1.f, 1.f, 1.f};
    if (NORM_Q) {
        const float *qsc = QFROMK ? sm.ks[pb] : sm.kq[pb];
        const float4 u4 = *reinterpret_cast<const float4 *>(&qsc[rb]);
        const float4 w4 = *reinterpret_cast<const float4 *>(&qsc[16 + rb]);
        qs0[0] = u4.x; qs0[1] = u4.y; qs0[2] = u4.z; qs0[3] = u4.w;
        qs1[0] = w4.x; qs1[1] = w4.y; qs1[2] = w4.z; qs1[3] = w4.w;
    }
    floatx4 x00, x10, x11;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = rb + j;
        const float e00 = exp2_(gt0[j] - g0) * (ks0 * qs0[j]) * P00[j];
        const float e11 = exp2_(gt1[j] - g1) * (ks1 * qs1[j]) * P11[j];
        x00[j] = c <= r ? e00 : 0.f;
        x10[j] = exp2_(gt1[j] - g0) * (ks0 * qs1[j]) * P10[j];
        x11[j] = c <= r ? e11 : 0.f;
    }
    _Float16 *pt = sm.pT[pb];
    *reinterpret_cast<half4 *>(&pt[c * C + rb]) = h4(x00);
    *reinterpret_cast<half4 *>(&pt[c * C + 16 + rb]) = h4(x10);
    *reinterpret_cast<half4 *>(&pt[(16 + c) * C + 16 + rb]) = h4(x11);
}

// Key-side tasks of one chunk after its conversion: wave 0 tile 0, wave 2
// tile 1, wave 3 A_10^T (kept in its registers, a10t, for its own combine),
// wave 1 P.
template <bool WANT_O, bool NORM_Q, bool QFROMK>
__device__ __forceinline__ void key_side_tasks(Smem &sm, int pb, int w, const Lane &L, floatx4 &a10t) {
    if (w == 1) {
        if (WANT_O) key_side_P<NORM_Q, QFROMK>(sm, pb, L);
        return;
    }
    if (w == 3) {
        a10t = key_side_a10t(sm, pb, L);
        return;
    }
    bool ill;
    const floatx4 r = key_side_tile(sm, pb, w >> 1, L, ill);
    key_side_tile_out(sm, w >> 1, r, ill, L);
}

// ---- state-side operand reads ---------------------------------------------------
// A fragment (rows t = lane%32, reduction s in the accumulator order of k-step
// ks) of a 32 x 32 fp16 matrix stored as (row s, column t) at LDS offset mat.
__device__ __forceinline__ half8 tr_frag_st(const Smem &sm, uint32_t mat, int ks, const Lane &L) {
    const uint32_t o = mat + L.st + 1024 * ks;
    return cat(tr4(sm, o), tr4(sm, o + 512));
}
// A fragment of K^T for state tile a (rows d_k = 32 a + lane%32) and k-step hf.
__device__ __forceinline__ half8 tr_frag_kt(const Smem &sm, uint32_t kbuf, int a, int hf, const Lane &L) {
    return cat(tr4(sm, kbuf + L.kt[hf][0] + 64 * a), tr4(sm, kbuf + L.kt[hf][1] + 64 * a));
}

// Store S = 2^{-sigma} Sacc (held as S^T tiles) to a d_v x d_k row-major block.
__device__ __forceinline__ void store_state(float *dst_head, const floatx16 (&Sacc)[4], float sigma, int w,
                                            int l32, int hi32) {
    float *dst = dst_head + (int64_t)(32 * w + l32) * DK;
    const float sc = exp2_(-sigma);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<float4 *>(dst + 32 * a + 8 * q4 + 4 * hi32) =
                make_float4(Sacc[a][4 * q4] * sc, Sacc[a][4 * q4 + 1] * sc, Sacc[a][4 * q4 + 2] * sc,
                            Sacc[a][4 * q4 + 3] * sc);
}

// Full token rows 8 w .. 8 w + 7 of a staged output tile (V buffer vbuf) to
// obase (the chunk's first row, head h, column 0); rows at or past lc are
// skipped.  Non-temporal: the outputs are not read again.
__device__ __forceinline__ void store_o_rows(const Smem &sm, int vbuf, gchar *obase, int lc, uint32_t hdv2, int w,
                                             const Lane &L) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const uint32_t tile = OFF_VR + (uint32_t)(vbuf * NW * C * 32 * 2);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const i16x4_t lo = tr4u(sm, tile + L.orr[k][0]), hi = tr4u(sm, tile + L.orr[k][1]);
        const u32x4 row = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        typedef __attribute__((address_space(1))) u32x4 gu32x4;
        gu32x4 *dst = (gu32x4 *)(obase + (size_t)(8 * w + 4 * k) * hdv2 + L.ost);
        if (lc == C || 8 * w + 4 * k + (L.n16 & 3) < lc) __builtin_nontemporal_store(row, dst);
    }
}

// One wave's part of a (request, head).  ROLE is the wave index: it selects
// the wave's value rows and key-side task, and as a compile-time constant it
// removes the per-chunk role branches.
// GROUP: one layer of a fused group launch, whose tensors and state slot come
// from lp instead of P (the requests, spans and flags are P's).
template <int ROLE, bool WANT_O, bool NORM_Q, bool ALIAS, bool SPLIT = false, bool GROUP = false>
__device__ __forceinline__ void wave_main(const LaunchDesc &P, Smem &sm, uint32_t sm_lds,
                                          const GroupLayer lp = GroupLayer{})
{
    // SPLIT (eight waves): waves 0-3 carry the state chain and waves 4-7 the
    // key side of the same schedule, each under role ROLE % 4; without SPLIT
    // every wave does both.  Both groups pass the same barriers.
    constexpr bool STATE = !SPLIT || ROLE < 4;
    constexpr bool KEY = !SPLIT || ROLE >= 4;
    // q = k = v, both normalised: the stored query rows are the stored key rows,
    // so the key tile and its scales serve as the query tile and query scales
    constexpr bool QFROMK = ALIAS && NORM_Q;

    const int Lg = xcd_remap(blockIdx.x, gridDim.x);
    const int h = Lg % P.H;
    const int r = Lg / P.H;
    const int b = P.req[r];
    const int H = P.H;
    int tid = threadIdx.x;
    // in a group launch, per layer: keeps the lane constants from being computed
    // once for all layers and held across them
    if (GROUP) asm volatile("" : "+v"(tid));
    constexpr int w = ROLE & 3;
    const Lane L = make_lane(tid, w, H);
    const int lane = L.lane, l32 = L.l32, hi32 = L.hi32;
    const int dv = 32 * w + l32;
    const int len = P.len[r];
    const int64_t row0 = P.row0[r];
    const int ne_end = P.emit_begin[r + 1];
    const int wf = P.wflags[r];
    const bool zero_v = (wf & kWorkZeroV) != 0;        // v = 0: no V copies, V tiles zero
    const bool out = WANT_O && !(wf & kWorkNoOut);      // outputs staged and stored
    Bases G;
    {
        const uint64_t th = (uint64_t)(row0 * H + h);  // token-head index of the span's first token
        G.ts = (uint32_t)(H * DK * 2);
        G.tg = (uint32_t)(H * 2);
        G.k = uniform64(reinterpret_cast<uint64_t>(GROUP ? lp.k : P.k) + th * (DK * 2));
        G.q = uniform64(reinterpret_cast<uint64_t>(GROUP ? lp.q : P.q) + th * (DK * 2));
        G.v = uniform64(reinterpret_cast<uint64_t>(GROUP ? lp.v : P.v) + th * (DV * 2) + 64 * w);
        G.o = uniform64(reinterpret_cast<uint64_t>(GROUP ? lp.o : P.o) + th * (DV * 2));
        G.a = uniform64(reinterpret_cast<uint64_t>(GROUP ? lp.alpha : P.alpha) + th * 2);
        G.b = uniform64(reinterpret_cast<uint64_t>(GROUP ? lp.beta : P.beta) + th * 2);
    }

    // ---- state S^T = 2^{-sigma} Sacc: tile a covers d_k rows 32a..32a+31; the
    // lane holds value row dv and d_k rows 8(j/4) + 4*hi32 + j%4 of each tile.
    floatx16 Sacc[4];
    float sigma = 0.f;  // S = 2^{-sigma} Sacc
    float mb = 0.f;     // bound on max |Sacc| per value column (lanes l, l ^ 32)
    if (!STATE) {
        // the key-side waves hold no state
    } else if (wf & kWorkIdentity) {
        // lane holds d_k rows 32 a + 8 (j/4) + 4 hi32 + j%4 of value row dv
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                Sacc[a][j] = (32 * a + 8 * (j >> 2) + 4 * hi32 + (j & 3)) == dv ? 1.f : 0.f;
    } else if (P.init_off[r] >= 0) {
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
    if (STATE && len > 0) {
        float mx = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(Sacc[a][j]));
        mx = wave_max(mx);
        if (mx > 0.f) {
            int E;
            frexpf(mx, &E);
            sigma = (float)(4 - E);
            const float sc = ldexpf(1.f, 4 - E);
#pragma unroll
            for (int a = 0; a < 4; ++a) Sacc[a] *= sc;
            mb = mx * sc;
        }
    }

    if (STATE && zero_v) {
        // both V buffers of this wave's columns stay zero (no copies, no output staging)
        typedef uint32_t u32x4z __attribute__((ext_vector_type(4)));
        const u32x4z zz = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int vbz = 0; vbz < NVB; ++vbz)
#pragma unroll
            for (int part = 0; part < 2; ++part)
                lds_st(sm, OFF_VR + (uint32_t)(((vbz * NW + w) * C * 32) * 2) + 1024 * part + 16 * lane, zz);
    }
    // The upper-right 16x16 blocks of T^T and P^T (s >= 16, t < 16) stay zero.
    for (int idx = tid; idx < 16 * 16; idx += NT) {
        const int o = (16 + (idx >> 4)) * C + (idx & 15);
        sm.tT[0][o] = sm.tT[1][o] = (_Float16)0.f;
        sm.pT[0][o] = sm.pT[1][o] = (_Float16)0.f;
    }

    Chunk cur;
    cur.t0 = 0;
    cur.ne = P.emit_begin[r];
    cur.lc = len > 0 ? chunk_len(P, len, 0, cur.ne, ne_end) : 0;
    Chunk nx = next_chunk(P, cur, len, ne_end);
    Pref pf;
    floatx4 a10t = {0.f, 0.f, 0.f, 0.f};  // wave 3 (key side): A_10^T of the chunk whose T is combined next
    int vb = 0;  // V buffer of the current chunk
    // With q = k = v (ALIAS) a chunk's rows are copied once, into raw tile
    // (chunk index % 2), and serve as keys, queries and values until the
    // copy of the chunk two ahead replaces them.
    constexpr uint32_t RAW1 = OFF_KQR + C * DK * 2;  // second raw tile
    if (KEY && cur.lc > 0) {
        if (!zero_v && !ALIAS) dma_v(sm_lds, 0, G, cur.t0, cur.lc, w, L);
        load_kq<0>(pf, sm_lds, G, cur.t0, cur.lc, w, L);
        load_kq<1, WANT_O && !ALIAS>(pf, sm_lds, G, cur.t0, cur.lc, w, L);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // the raw rows of chunk 0 have landed (each wave its own copies)
    }
    lds_barrier();
    if (cur.lc > 0) {
        if (KEY) {
            if (ALIAS) key_side_convert<WANT_O && !QFROMK, NORM_Q, w, 4, SPLIT>(sm, 0, pf, cur.lc, L, OFF_KQR, OFF_KQR);
            else key_side_convert<WANT_O, NORM_Q, w, 4, SPLIT>(sm, 0, pf, cur.lc, L);
        }
        lds_barrier();  // the raw tiles are free again (ALIAS: tile 0 keeps chunk 0's values)
        if (KEY && nx.lc > 0) {
            load_kq<0>(pf, sm_lds, G, nx.t0, nx.lc, w, L, ALIAS ? RAW1 : OFF_KQR);
            load_kq<1, WANT_O && !ALIAS>(pf, sm_lds, G, nx.t0, nx.lc, w, L);
        }
        if (KEY) key_side_tasks<WANT_O, NORM_Q, QFROMK>(sm, 0, w, L, a10t);
    }

    int p = 0;   // key-side buffer of the current chunk
    int kp = 0;  // ALIAS: raw tile of the current chunk
    // outputs of the previous chunk, staged in V buffer vb_pend, are stored after the next barrier
    gchar *obase_pend = nullptr;
    int lc_pend = 0, vb_pend = 0;
    while (cur.lc > 0) {
        const Chunk nx2 = next_chunk(P, nx, len, ne_end);
        // raw keys of `nx2` before the task, queries (and gates) after it; all
        // before the output stores (see the wait below)
        const bool has2 = nx2.lc > 0;
        const int kt2 = has2 ? nx2.t0 : cur.t0;
        const int klc2 = has2 ? nx2.lc : cur.lc;
        // eight waves, separate tensors: each key-side wave copies the rows it
        // converts, as soon as its own conversion has read them
        constexpr bool EARLY = SPLIT && !ALIAS;
        // every load this wave issued has landed; the barrier then publishes the
        // raw key/query rows and the staged outputs to all waves
        __builtin_amdgcn_s_waitcnt(0x0F70);
        lds_barrier();  // key-side tasks of `cur` complete; previous state step done
        if (WANT_O && lc_pend > 0) {
            if (STATE) store_o_rows(sm, vb_pend, obase_pend, lc_pend, G.ts, w, L);
            lc_pend = 0;
        }
        // ---- state side of `cur` ------------------------------------------------
        const int lc = cur.lc;
        const uint32_t kbuf = OFF_KH + p * KBUF;  // keys of `cur`; queries at + 2 KBUF
        const uint32_t cw = L.cwr;                 // cw[w][j][8 q4 + 4 hi32 ..] at cw + 128 j + 32 q4
        float *cwl = sm.cw[w][0];

        // key side of `nx`: conversion (independent of the state chain above)
        if (KEY && nx.lc > 0) {
            if (ALIAS) {
                const uint32_t rawn = kp ? OFF_KQR : RAW1;  // raw tile of `nx`
                key_side_convert<WANT_O && !QFROMK, NORM_Q, w, 4, SPLIT>(sm, p ^ 1, pf, nx.lc, L, rawn, rawn);
            } else {
                key_side_convert<WANT_O, NORM_Q, w, 4, SPLIT>(sm, p ^ 1, pf, nx.lc, L);
            }
        }
        if (EARLY && KEY) {
            load_owned<WANT_O, w>(sm_lds, G, kt2, klc2, L);
            load_kq<1, false>(pf, sm_lds, G, kt2, klc2, w, L);  // gates of `nx2`
        }
        floatx16 Y = {}, Z = {};
        int eB = 0;
        if (STATE) {
        // Y = K^ Sacc^T and Z = Q^ Sacc^T (Sacc within the fp16 band by construction)
        // (all fragments are read first, so that the reads overlap)
        half8 kf[8], qf[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            kf[m] = lds_ld<half8>(sm, kbuf + L.yz + 32 * m);
            if (WANT_O) qf[m] = lds_ld<half8>(sm, kbuf + (QFROMK ? 0 : 2 * KBUF) + L.yz + 32 * m);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const half8 sf = to_frag(Sacc[m >> 1], m & 1);
            Y = mfma32(kf[m], sf, Y);
            if (WANT_O) Z = mfma32(qf[m], sf, Z);
        }
        // schedule: all reads, then per step the fragment conversion and the products
#pragma unroll
        for (int i = 0; i < (WANT_O ? 16 : 8); ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, WANT_O ? 2 : 1, 0);
        }
        const float isg = exp2_(-sigma);
        if (lane < 32) {
            const float e = sm.eg[p][lane];      // 2^{g_t}
            const float kst = sm.ks[p][lane];    // k^_t = kst k'_t
            const float kq = QFROMK ? kst : sm.kq[p][lane];  // q^_t (or q_t) = kq q'_t
            cwl[lane] = e * isg * kst;           // B~ = v - cw0 Y', Y' = K' Sacc^T
            if (WANT_O) cwl[C + lane] = kq * e * isg;  // o (state part) = cw1 Z
            // W' = cw2 U (rows of K'^T W' = K^^T W) and o (intra part) = cw3 (P U'),
            // for unscaled T, B~, U and no rescale of the state (rewritten below
            // otherwise): 2^{g_C - g_t} 2^{sigma - g_C} kst
            cwl[2 * C + lane] = sm.ws[p][lane] * exp2_(sigma - sm.gl[p][C - 1]) * kst;
            if (WANT_O && !NORM_Q) cwl[3 * C + lane] = kq;
        }
        // B~ = v - 2^{g_t} S_0 k^_t, in place in Y
        float bm = 0.f;
        {
            // values: the wave's V slice (64-byte token rows), or with ALIAS the
            // raw tile of `cur` (256-byte rows); zero-v works keep the zeroed slices
            const bool rawv = ALIAS && !zero_v;
            const uint32_t vbase = rawv ? (kp ? RAW1 : OFF_KQR) + L.vrdr
                                        : OFF_VR + (uint32_t)((vb * NW + w) * C * 32 * 2) + L.vrd;
            const uint32_t vstep = rawv ? 8 * DK * 2 : 512;  // 8 tokens
            i16x4_t vv[4];
            float4 c4[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                vv[q4] = tr4u(sm, vbase + vstep * q4);
                c4[q4] = lds_ld<float4>(sm, cw + 32 * q4);
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float cc[4] = {c4[q4].x, c4[q4].y, c4[q4].z, c4[q4].w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float x = bf((uint16_t)vv[q4][jj]) - cc[jj] * Y[4 * q4 + jj];
                    Y[4 * q4 + jj] = x;
                    bm = fmaxf(bm, fabsf(x));
                }
            }
        }
        if (out_of_band(bm)) eB = f16_adjust(wave_max(bm));
        if (eB != 0) Y *= ldexpf(1.f, eB);
        }  // STATE
        if (KEY && w == 3) {
            // the last T step is on the critical path of this phase: it takes
            // issue priority over the co-resident workgroup's waves
            __builtin_amdgcn_s_setprio(2);
            key_side_combine(sm, p, L, a10t);
            __builtin_amdgcn_s_setprio(0);
        }
        lds_barrier();  // T of `cur` and the keys of `nx` are complete
        auto key_phase = [&]() {
            if (!EARLY && w == 3) load_k_all(sm_lds, G, kt2, klc2, L, ALIAS ? (kp ? RAW1 : OFF_KQR) : OFF_KQR);
            // V of `nx` into the other V buffer (its staged outputs went out after the
            // first barrier; without a next chunk, rows of `cur` are copied and ignored)
            if (!zero_v && !ALIAS && w == 3) {
                const bool has1 = nx.lc > 0;
                dma_v_all(sm_lds, vb ^ 1, G, has1 ? nx.t0 : cur.t0, has1 ? nx.lc : cur.lc, L);
            }
            if (w != 3) __builtin_amdgcn_s_setprio(1);  // the longer tasks of this phase go first
            if (nx.lc > 0) key_side_tasks<WANT_O, NORM_Q, QFROMK>(sm, p ^ 1, w, L, a10t);
            if (w != 3) __builtin_amdgcn_s_setprio(0);
            if (!EARLY) load_kq<1, WANT_O && !ALIAS>(pf, sm_lds, G, kt2, klc2, w, L);
        };
        if (SPLIT && KEY) key_phase();
        if (STATE) {
        // operands of `cur` that are complete now are read before the tasks
        const half8 tfr0 = tr_frag_st(sm, OFF_TT, 0, L);
        const half8 tfr1 = tr_frag_st(sm, OFF_TT, 1, L);
        // lo part of T: zero unless the combine took the hi/lo form
        const bool tlo = sm.tlo != 0;
        half8 tfl0, tfl1;
        if (tlo) {
            tfl0 = tr_frag_st(sm, OFF_TT + C * C * 2, 0, L);
            tfl1 = tr_frag_st(sm, OFF_TT + C * C * 2, 1, L);
        }
        half8 pfr0, pfr1;
        if (WANT_O) {
            pfr0 = tr_frag_st(sm, OFF_PT + p * (C * C * 2), 0, L);
            pfr1 = tr_frag_st(sm, OFF_PT + p * (C * C * 2), 1, L);
        }
        const float tsc = sm.tsc;
        const float gCp = sm.gl[p][C - 1];
        if (!SPLIT) key_phase();
        // the rest of phase two goes first: before the co-resident workgroup's phase
        // one (four waves), before the key-side waves of the same workgroup (eight)
        __builtin_amdgcn_s_setprio(1);

        // U = (T diag(beta)) B~, T as its hi/lo pair
        floatx16 U = {};
        const half8 yf0 = to_frag(Y, 0), yf1 = to_frag(Y, 1);
        U = mfma32(tfr0, yf0, U);
        U = mfma32(tfr1, yf1, U);
        if (tlo) {
            U = mfma32(tfl0, yf0, U);
            U = mfma32(tfl1, yf1, U);
        }
        // K^T fragments of the state update
        half8 ktf[4][2];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) ktf[a][hf] = tr_frag_kt(sm, kbuf, a, hf, L);
        float um = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) um = fmaxf(um, fabsf(U[j]));
        int eU = 0;
        if (out_of_band(um)) eU = f16_adjust(wave_max(um));
        int ets;
        frexpf(tsc, &ets);
        const float lus = (float)(ets - 1 - eB);  // u = us U with us = tsc 2^-eB = 2^lus

        // scale of the new state: decay folded into sigma; rescale Sacc only
        // when the bound on max |Sacc| would leave [1, 2^14], or when the state
        // exponent would exceed kSigMax (a decaying state with nothing written,
        // e.g. v = 0 or tiny gates; without the cap 2^sigma would overflow).
        // The bound is kept per value column (lanes l and l ^ 32 hold the
        // column's tokens): |K^T W'| <= 32 max|W'|, max|W'| <= max|U| us 2^sig1,
        // evaluated in log2 so that no intermediate power of two overflows.
        float sig1 = sigma - gCp;
        const float umx = fmaxf(um, partner32(um, lane));
        const float linc = 5.f + log2_(umx) + lus + sig1;  // log2 of the bound (-inf when U = 0)
        const float dmin = fmaxf(sig1 - kSigMax, 0.f);     // forced shift
        const float mbn = mb * exp2_(-dmin) + exp2_(fminf(linc - dmin, 127.f));
        float delta = dmin;
        if (__builtin_amdgcn_ballot_w64(mbn > 0x1p14f) != 0 ||
            (__builtin_amdgcn_ballot_w64(mbn >= 1.f) == 0 && __builtin_amdgcn_ballot_w64(mbn > 0.f) != 0)) {
            float mx = 0.f;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(Sacc[a][j]));
            // log2(max|Sacc| + max incl) at exponent sig1, then the shift that
            // brings it to [8, 16), but never below the forced one
            const float lm = log2_(wave_max(mx)), li = wave_max(linc);
            const float hi = fmaxf(lm, li), lo = fminf(lm, li);
            const float ltot = lo > -INFINITY ? hi + log2_(1.f + exp2_(lo - hi)) : hi;  // -inf: all zero
            delta = fmaxf(floorf(ltot) - 3.f, sig1 - kSigMax);
            mb = exp2_(ltot - delta);
        } else {
            mb = mbn;
        }
        sig1 -= delta;
        const float dsc = exp2_(fminf(-delta, 126.f));  // Sacc is zero whenever -delta would be larger
        const bool scaled = tsc != 1.f || eB != 0 || eU != 0 || delta != 0.f;
        if (scaled && lane < 32) {
            // W' = cw2 U, cw2 = 2^{g_C - g_t} 2^sig1 us as one power of two
            cwl[2 * C + lane] = exp2_(fminf(gCp - sm.gl[p][lane] + sig1 + lus, 126.f)) * sm.ks[p][lane];
            if (WANT_O) cwl[3 * C + lane] = (NORM_Q ? 1.f : sm.kq[p][lane]) * exp2_(lus - (float)eU);  // o (intra) = cw3 (P U')
        }

        if (WANT_O) {
            half8 Uf0 = to_frag(U, 0), Uf1 = to_frag(U, 1);
            if (eU != 0) {
                const floatx16 Us = U * ldexpf(1.f, eU);
                Uf0 = to_frag(Us, 0);
                Uf1 = to_frag(Us, 1);
            }
            floatx16 PO = {};
            PO = mfma32(pfr0, Uf0, PO);
            PO = mfma32(pfr1, Uf1, PO);
            float ov[16];
            // the intra-chunk part needs no coefficient when q is normalised and
            // T, B~ and U are unscaled
            if (NORM_Q && !scaled) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 z4 = lds_ld<float4>(sm, cw + 128 + 32 * q4);
                    const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) ov[4 * q4 + jj] = zz[jj] * Z[4 * q4 + jj] + PO[4 * q4 + jj];
                }
            } else {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 z4 = lds_ld<float4>(sm, cw + 128 + 32 * q4);
                    const float4 p4 = lds_ld<float4>(sm, cw + 384 + 32 * q4);
                    const float zz[4] = {z4.x, z4.y, z4.z, z4.w}, pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        ov[4 * q4 + jj] = zz[jj] * Z[4 * q4 + jj] + pp[jj] * PO[4 * q4 + jj];
                }
            }
            // o_t into the chunk's output tile (the V buffer, consumed by every
            // wave's B~); full rows go out after the next barrier
            if (out) {
                const uint32_t tile = OFF_VR + (uint32_t)(vb * NW * C * 32 * 2);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    lds_st(sm, tile + L.ow[q4], make_uint2(pack_bf16(ov[4 * q4], ov[4 * q4 + 1]),
                                                           pack_bf16(ov[4 * q4 + 2], ov[4 * q4 + 3])));
                obase_pend = (gchar *)at_tok(G.o, cur.t0, G.ts);  // wave-uniform
                lc_pend = lc;
                vb_pend = vb;
            }
        }
        // W' = 2^{sig1} 2^{g_C - g_s} u_s (Sacc units), then Sacc <- Sacc 2^{-delta} + K^ T W'
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 s4 = lds_ld<float4>(sm, cw + 256 + 32 * q4);
            U[4 * q4 + 0] *= s4.x;
            U[4 * q4 + 1] *= s4.y;
            U[4 * q4 + 2] *= s4.z;
            U[4 * q4 + 3] *= s4.w;
        }
        const half8 Wf0 = to_frag(U, 0), Wf1 = to_frag(U, 1);
        if (delta != 0.f) {
#pragma unroll
            for (int a = 0; a < 4; ++a) Sacc[a] *= dsc;
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            Sacc[a] = mfma32(ktf[a][0], Wf0, Sacc[a]);
            Sacc[a] = mfma32(ktf[a][1], Wf1, Sacc[a]);
        }
        sigma = sig1;

        if (cur.ne < ne_end && P.emit_after[cur.ne] == cur.t0 + lc)
            store_state(P.emit_base + (((int64_t)b * P.M + P.emit_slot[cur.ne]) * H + h) * DV * DK, Sacc, sigma,
                        w, l32, hi32);
        }  // STATE
        if (STATE) __builtin_amdgcn_s_setprio(0);
        if (SPLIT && !STATE && out) lc_pend = lc;  // the key-side waves pass the same final barrier
        cur = nx;
        nx = nx2;
        p ^= 1;
        vb ^= 1;
        kp ^= 1;
    }

    if (WANT_O && lc_pend > 0) {
        lds_barrier();  // the last staged outputs are complete
        if (STATE) store_o_rows(sm, vb_pend, obase_pend, lc_pend, G.ts, w, L);
    }
    if (STATE && P.state_dst[r])
        store_state(P.state_dst[r] + (GROUP ? lp.state_shift : 0) + (int64_t)h * DV * DK, Sacc, sigma, w, l32, hi32);
}

// ---- d_v in two halves --------------------------------------------------------
// A launch that leaves half of the CUs idle gives each (request, head) two
// workgroups of eight waves, one per half of its d_v = 128 value rows: the
// rows of S do not interact (the key operator of eq. (1) acts from the right).
// Waves 4-7 run the key side exactly as the eight-wave kernel does (both
// halves form the same T and P; their key and gate rows are read by two
// workgroups of one XCD).  Waves 0-3 each own 16 value rows of the half and
// run the state side on v_mfma_f32_16x16x32_f16, so that each wave's share of
// every state product is half that of the eight-wave kernel.
//
// State wave w of half hv, lane (g, n) = (lane / 16, lane % 16), value row
// dvr = 64 hv + 16 w + n:
//  - S^T is held as 8 accumulator tiles of 16 stored key columns; tile a,
//    accumulator row 4 g' + j covers the stored column 32 (a/2) + 8 g' + 4 (a%2) + j,
//    so that tiles 2m and 2m+1 of a lane make one 8-element B fragment of the
//    stored columns 32 m + 8 g .. +7, i.e. one 16-byte read of a key row;
//  - Y = K S^T, B~, U and W' (lane: value column n, tokens 16 tb + 4 g + j);
//    Z^T = S Q^T and O^T (lane: token 16 tt + n, value columns 4 g + j), so
//    that a lane stores 4 consecutive outputs as 8 bytes;
//  - K^T, T and P as A / B operands in the token order of U's tiles (s = 4 g + j
//    and 16 + 4 g + j) come from transposed reads of the token-major tiles.
// V of a chunk: 32 rows of the half's 64 columns (128 bytes) per buffer, the
// 16-byte slot u of row t holding the row's unit u ^ 2 ((t / 2) % 4) (the
// transposed B~ reads are then free of bank conflicts).
constexpr uint32_t V2BUF = C * 128;  // bytes of one V buffer
static_assert(NVB * V2BUF <= sizeof(Smem::vr), "V buffers of the split kernel fit the V staging area");

struct Lane2 {
    uint32_t yz;     // Y / Z fragments: row krow(n), stored column 8 g (+64 bytes per k-step, +16 rows per token tile)
    uint32_t vrd;    // transposed V reads of token tile 0 (+2048 bytes for tile 1)
    uint32_t st;     // transposed T / P reads of s = 4 g + (n / 4), t = 4 (n % 4) (+32 bytes per t tile, +1024 for s + 16)
    uint32_t kt[2];  // transposed K^T reads, s = 4 g + n / 4 (+16 for kt[1]), stored column 8 (n % 4)
    uint32_t vcol;   // V copies: the lane's 16-byte unit of a row (swizzled)
    int scol;        // logical key column of accumulator row 4 g of tile 0 (+32 (a/2) + 8 (a%2))
};
__device__ __forceinline__ Lane2 make_lane2(int lane, int w) {
    const int g = lane >> 4, n = lane & 15;
    Lane2 L;
    L.yz = krow(n) * KROWB + 16 * g;
    L.vrd = (4 * g + (n >> 2)) * 128 + 16 * ((2 * w + ((n & 3) >> 1)) ^ (2 * ((2 * g + (n >> 3)) & 3))) + 8 * (n & 1);
    L.st = (4 * g + (n >> 2)) * 64 + 8 * (n & 3);
    L.kt[0] = krow(4 * g + (n >> 2)) * KROWB + 16 * (n & 3);
    L.kt[1] = krow(16 + 4 * g + (n >> 2)) * KROWB + 16 * (n & 3);
    L.vcol = 16 * ((lane & 7) ^ (2 * ((lane >> 4) & 3)));
    // stored column 32 m + 8 g + 4 h + j is the key column 32 m + 16 (g/2) + 8 h + 4 (g%2) + j
    L.scol = 16 * (g >> 1) + 4 * (g & 1);
    return L;
}

// V rows 8 i .. 8 i + 7 of a chunk into buffer vb (1 KiB): lane l writes slot
// l % 8 of row 8 i + l / 8.  Rows past the chunk are clamped to its last row.
__device__ __forceinline__ void dma_v2(uint32_t sm_lds, int vb, const Bases &G, int t0, int lc, const Lane2 &L2,
                                       int lane, int i) {
    const uint64_t base = at_tok(G.v, t0, G.ts);
    const uint32_t lim = (uint32_t)(lc - 1) * G.ts + L2.vcol;
    dma16(base, min((uint32_t)(8 * i + (lane >> 3)) * G.ts + L2.vcol, lim),
          sm_lds + OFF_VR + (uint32_t)(vb * V2BUF + 1024 * i));
}

// S = 2^{-sigma} S2 of value row dvr to a d_v x d_k row-major block.
__device__ __forceinline__ void store_state2(float *dst_head, const floatx4 (&S2)[8], float sigma, int dvr, int scol) {
    float *dst = dst_head + (int64_t)dvr * DK + scol;
    const float sc = exp2_(-sigma);
#pragma unroll
    for (int a = 0; a < 8; ++a)
        *reinterpret_cast<float4 *>(dst + 32 * (a >> 1) + 8 * (a & 1)) =
            make_float4(S2[a][0] * sc, S2[a][1] * sc, S2[a][2] * sc, S2[a][3] * sc);
}

// A fragment of a 32 x 32 fp16 matrix X stored as (row s, column t): rows
// t = 16 tt + n, reduction s in the order 4 g + j, 16 + 4 g + j.
__device__ __forceinline__ half8 tr_frag2(const Smem &sm, uint32_t mat, int tt, const Lane2 &L2) {
    const uint32_t o = mat + L2.st + 32 * tt;
    return cat(tr4(sm, o), tr4(sm, o + 1024));
}

// Tile tasks of a chunk with NK key-side waves (role kr): tile 0 on role 0,
// tile 1 on role 2, P on role 1, A_10 on the role that finishes T (kept in
// its registers for the combine).
template <bool WANT_O, bool NORM_Q, int NK>
__device__ __forceinline__ void dv2_key_tasks(Smem &sm, int pb, int kr, const Lane &L, floatx4 &a10t) {
    if (kr == 1) {
        if (WANT_O) key_side_P<NORM_Q, false>(sm, pb, L);
    } else if (kr == NK - 1) {
        a10t = key_side_a10t(sm, pb, L);
    } else if (kr == 0 || kr == 2) {
        bool ill;
        const floatx4 t = key_side_tile(sm, pb, kr >> 1, L, ill);
        key_side_tile_out(sm, kr >> 1, t, ill, L);
    }
}

template <int ROLE, bool WANT_O, bool NORM_Q, int NK>
__device__ __forceinline__ void dv2_main(const LaunchDesc &P, Smem &sm, uint32_t sm_lds)
{
    constexpr bool STATE = ROLE < 4;
    constexpr bool KEY = ROLE >= 4;
    constexpr int kr = ROLE - 4;                // key-side role (0 .. NK - 1)
    constexpr int w = KEY ? (kr & 3) : ROLE;    // lane constants of the four-wave layout
    constexpr int KC = NK - 1;                  // key-side role that finishes T

    const int Lg = xcd_remap(blockIdx.x, gridDim.x);
    const int hv = Lg & 1;
    const int pair = Lg >> 1;
    const int h = pair % P.H;
    const int r = pair / P.H;
    const int b = P.req[r];
    const int H = P.H;
    const int tid = threadIdx.x;
    const Lane L = make_lane(tid, w, H);
    const Lane2 L2 = make_lane2(L.lane, w);
    const int lane = L.lane, g = L.g, n = L.n16;
    const int dvr = 64 * hv + 16 * w + n;
    const int len = P.len[r];
    const int64_t row0 = P.row0[r];
    const int ne_end = P.emit_begin[r + 1];
    const int wf = P.wflags[r];
    const bool zero_v = (wf & kWorkZeroV) != 0;
    const bool out = WANT_O && !(wf & kWorkNoOut);
    Bases G;
    {
        const uint64_t th = (uint64_t)(row0 * H + h);
        G.ts = (uint32_t)(H * DK * 2);
        G.tg = (uint32_t)(H * 2);
        G.k = uniform64(reinterpret_cast<uint64_t>(P.k) + th * (DK * 2));
        G.q = uniform64(reinterpret_cast<uint64_t>(P.q) + th * (DK * 2));
        G.v = uniform64(reinterpret_cast<uint64_t>(P.v) + th * (DV * 2) + 128 * hv);
        G.o = uniform64(reinterpret_cast<uint64_t>(P.o) + th * (DV * 2) + 128 * hv);
        G.a = uniform64(reinterpret_cast<uint64_t>(P.alpha) + th * 2);
        G.b = uniform64(reinterpret_cast<uint64_t>(P.beta) + th * 2);
    }

    floatx4 S2[8];
    float sigma = 0.f;
    float mb = 0.f;  // bound on max |S2| per value column (lanes n, n + 16, n + 32, n + 48)
    if (!STATE) {
    } else if (wf & kWorkIdentity) {
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j) S2[a][j] = (32 * (a >> 1) + 8 * (a & 1) + L2.scol + j) == dvr ? 1.f : 0.f;
    } else if (P.init_off[r] >= 0) {
        const float *src = P.init_base + P.init_off[r] + (int64_t)h * DV * DK + (int64_t)dvr * DK + L2.scol;
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            const float4 v4 = *reinterpret_cast<const float4 *>(src + 32 * (a >> 1) + 8 * (a & 1));
            S2[a][0] = v4.x;
            S2[a][1] = v4.y;
            S2[a][2] = v4.z;
            S2[a][3] = v4.w;
        }
    } else {
#pragma unroll
        for (int a = 0; a < 8; ++a) S2[a] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    if (STATE && len > 0) {
        float mx = 0.f;
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fabsf(S2[a][j]));
        mx = wave_max(mx);
        if (mx > 0.f) {
            int E;
            frexpf(mx, &E);
            sigma = (float)(4 - E);
            const float sc = ldexpf(1.f, 4 - E);
#pragma unroll
            for (int a = 0; a < 8; ++a) S2[a] *= sc;
            mb = mx * sc;
        }
    }
    if (STATE && zero_v) {
        // both V buffers stay zero (no copies)
        typedef uint32_t u32x4z __attribute__((ext_vector_type(4)));
        const u32x4z zz = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int part = 0; part < 2; ++part) lds_st(sm, OFF_VR + (uint32_t)(2048 * w + 1024 * part) + 16 * lane, zz);
    }
    for (int idx = tid; idx < 16 * 16; idx += NT) {
        const int o = (16 + (idx >> 4)) * C + (idx & 15);
        sm.tT[0][o] = sm.tT[1][o] = (_Float16)0.f;
        sm.pT[0][o] = sm.pT[1][o] = (_Float16)0.f;
    }

    Chunk cur;
    cur.t0 = 0;
    cur.ne = P.emit_begin[r];
    cur.lc = len > 0 ? chunk_len(P, len, 0, cur.ne, ne_end) : 0;
    Chunk nx = next_chunk(P, cur, len, ne_end);
    Pref pf;
    floatx4 a10t = {0.f, 0.f, 0.f, 0.f};
    int vb = 0;
    // each key-side role copies the raw rows it converts (and role 1 the gates)
    if (KEY && cur.lc > 0) {
        if (!zero_v && kr < 4) dma_v2(sm_lds, 0, G, cur.t0, cur.lc, L2, lane, kr);
        load_owned<WANT_O, kr, NK>(sm_lds, G, cur.t0, cur.lc, L);
        load_kq<1, false>(pf, sm_lds, G, cur.t0, cur.lc, kr == 1 ? 1 : 0, L);
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    lds_barrier();
    if (cur.lc > 0) {
        if (KEY) key_side_convert<WANT_O, NORM_Q, kr, NK, true>(sm, 0, pf, cur.lc, L);
        lds_barrier();
        if (KEY && nx.lc > 0) {
            load_owned<WANT_O, kr, NK>(sm_lds, G, nx.t0, nx.lc, L);
            load_kq<1, false>(pf, sm_lds, G, nx.t0, nx.lc, kr == 1 ? 1 : 0, L);
        }
        if (KEY) dv2_key_tasks<WANT_O, NORM_Q, NK>(sm, 0, kr, L, a10t);
    }

    int p = 0;
    while (cur.lc > 0) {
        const Chunk nx2 = next_chunk(P, nx, len, ne_end);
        const bool has2 = nx2.lc > 0;
        const int kt2 = has2 ? nx2.t0 : cur.t0;
        const int klc2 = has2 ? nx2.lc : cur.lc;
        // the key-side waves' copies have landed (the state waves issue no loads)
        if (KEY) __builtin_amdgcn_s_waitcnt(0x0F70);
        lds_barrier();  // key-side tasks of `cur` complete; previous state step done
        const int lc = cur.lc;
        const uint32_t kbuf = OFF_KH + p * KBUF;
        const uint32_t cwb = OFF_CW + (uint32_t)(w * 4 * C * 4);  // this wave's coefficient rows
        // key side of `nx`: conversion, then the raw rows of `nx2` that this
        // wave converts next (and the gates)
        if (KEY && nx.lc > 0) key_side_convert<WANT_O, NORM_Q, kr, NK, true>(sm, p ^ 1, pf, nx.lc, L);
        if (KEY) {
            load_owned<WANT_O, kr, NK>(sm_lds, G, kt2, klc2, L);
            load_kq<1, false>(pf, sm_lds, G, kt2, klc2, kr == 1 ? 1 : 0, L);  // gates of `nx2`
        }

        floatx4 Y2[2], Z2[2];
        int eB = 0;
        // coefficients of this chunk read back in phase one (rewritten in the
        // rare scaled case): o = zc Z + pc (P U'), W' = c2 U, and g_C
        float zc[2], pc[2], gCp;
        floatx4 c2[2];
        if (STATE) {
            // Y = K^ S2^T, Z^T = S2 Q^T: all fragments first, so that the reads overlap
            half8 kf[2][4], qf[2][4];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    kf[tb][m] = lds_ld<half8>(sm, kbuf + L2.yz + 16 * KROWB * tb + 64 * m);
                    if (WANT_O) qf[tb][m] = lds_ld<half8>(sm, kbuf + 2 * KBUF + L2.yz + 16 * KROWB * tb + 64 * m);
                }
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) Y2[tb] = Z2[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const half8 sf = cat(h4(S2[2 * m]), h4(S2[2 * m + 1]));
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    Y2[tb] = mfma16(kf[tb][m], sf, Y2[tb]);
                    if (WANT_O) Z2[tb] = mfma16(sf, qf[tb][m], Z2[tb]);
                }
            }
            const float isg = exp2_(-sigma);
            float *cwl = sm.cw[w][0];
            if (lane < 32) {
                const float e = sm.eg[p][lane];
                const float kst = sm.ks[p][lane];
                const float kq = sm.kq[p][lane];
                cwl[lane] = e * isg * kst;       // B~ = v - cw0 Y'
                if (WANT_O) cwl[C + lane] = kq * e * isg;  // o (state part) = cw1 Z
                cwl[2 * C + lane] = sm.ws[p][lane] * exp2_(sigma - sm.gl[p][C - 1]) * kst;  // W' = cw2 U
                if (WANT_O && !NORM_Q) cwl[3 * C + lane] = kq;  // o (intra part) = cw3 (P U')
            }
            gCp = sm.gl[p][C - 1];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                if (WANT_O) zc[tt] = cwl[C + 16 * tt + n];
                pc[tt] = (WANT_O && !NORM_Q) ? cwl[3 * C + 16 * tt + n] : 1.f;
                c2[tt] = lds_ld<floatx4>(sm, cwb + 4 * (2 * C + 16 * tt + 4 * g));
            }
            // B~ = v - 2^{g_t} S_0 k^_t, in place in Y
            float bm = 0.f;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const i16x4_t vv = tr4u(sm, OFF_VR + (uint32_t)(vb * V2BUF) + 2048 * tb + L2.vrd);
                const float4 c4 = lds_ld<float4>(sm, cwb + 4 * (16 * tb + 4 * g));
                const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x = bf((uint16_t)vv[j]) - cc[j] * Y2[tb][j];
                    Y2[tb][j] = x;
                    bm = fmaxf(bm, fabsf(x));
                }
            }
            if (out_of_band(bm)) eB = f16_adjust(wave_max(bm));
            if (eB != 0) {
                const float sc = ldexpf(1.f, eB);
                Y2[0] *= sc;
                Y2[1] *= sc;
            }
        }
        if (KEY && kr == KC) {
            __builtin_amdgcn_s_setprio(2);
            key_side_combine(sm, p, L, a10t);
            __builtin_amdgcn_s_setprio(0);
        }
        lds_barrier();  // T of `cur` and the keys of `nx` are complete
        if (KEY) {
            // V of `nx` into the other buffer (last read by the B~ of the previous chunk)
            if (!zero_v && kr == 3) {
                const bool has1 = nx.lc > 0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dma_v2(sm_lds, vb ^ 1, G, has1 ? nx.t0 : cur.t0, has1 ? nx.lc : cur.lc, L2, lane, i);
            }
            if (nx.lc > 0) dv2_key_tasks<WANT_O, NORM_Q, NK>(sm, p ^ 1, kr, L, a10t);
        }
        if (STATE) {
            // the state chain is the longer side of this phase: it takes issue
            // priority over the tile tasks (which have slack until the barrier)
            __builtin_amdgcn_s_setprio(1);
            const float tsc = sm.tsc;
            const half8 th0 = tr_frag2(sm, OFF_TT, 0, L2), th1 = tr_frag2(sm, OFF_TT, 1, L2);
            const bool tlo = sm.tlo != 0;  // T has a lo part (the combine took the hi/lo form)
            half8 tl0, tl1;
            if (tlo) {
                tl0 = tr_frag2(sm, OFF_TT + C * C * 2, 0, L2);
                tl1 = tr_frag2(sm, OFF_TT + C * C * 2, 1, L2);
            }
            half8 pf0, pf1;
            if (WANT_O) {
                pf0 = tr_frag2(sm, OFF_PT + p * (C * C * 2), 0, L2);
                pf1 = tr_frag2(sm, OFF_PT + p * (C * C * 2), 1, L2);
            }
            // U = (T diag(beta)) B~, T as its hi/lo pair
            const half8 bfr = cat(h4(Y2[0]), h4(Y2[1]));
            floatx4 U2[2];
            U2[0] = mfma16(th0, bfr, floatx4{0.f, 0.f, 0.f, 0.f});
            U2[1] = mfma16(th1, bfr, floatx4{0.f, 0.f, 0.f, 0.f});
            if (tlo) {
                U2[0] = mfma16(tl0, bfr, U2[0]);
                U2[1] = mfma16(tl1, bfr, U2[1]);
            }
            half8 ktf[8];
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                const uint32_t co = 64 * (a >> 1) + 8 * (a & 1);
                ktf[a] = cat(tr4(sm, kbuf + L2.kt[0] + co), tr4(sm, kbuf + L2.kt[1] + co));
            }
            float um = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) um = fmaxf(um, fmaxf(fabsf(U2[0][j]), fabsf(U2[1][j])));
            int eU = 0;
            if (out_of_band(um)) eU = f16_adjust(wave_max(um));
            int ets;
            frexpf(tsc, &ets);
            const float lus = (float)(ets - 1 - eB);  // u = us U with us = tsc 2^-eB = 2^lus

            // scale of the new state (the rule of the four-wave kernel; a value
            // column's tokens sit in lanes n, n + 16, n + 32, n + 48)
            float sig1 = sigma - gCp;
            float umx;
            {
                // maxima over lane pairs (l, l ^ 16), then (l, l ^ 32)
                const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(um), __float_as_uint(um), false, false);
                umx = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
                const auto b2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(umx), __float_as_uint(umx), false, false);
                umx = fmaxf(__uint_as_float(b2[0]), __uint_as_float(b2[1]));
            }
            const float linc = 5.f + log2_(umx) + lus + sig1;
            const float dmin = fmaxf(sig1 - kSigMax, 0.f);
            const float mbn = mb * exp2_(-dmin) + exp2_(fminf(linc - dmin, 127.f));
            float delta = dmin;
            if (__builtin_amdgcn_ballot_w64(mbn > 0x1p14f) != 0 ||
                (__builtin_amdgcn_ballot_w64(mbn >= 1.f) == 0 && __builtin_amdgcn_ballot_w64(mbn > 0.f) != 0)) {
                float mx = 0.f;
#pragma unroll
                for (int a = 0; a < 8; ++a)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fabsf(S2[a][j]));
                const float lm = log2_(wave_max(mx)), li = wave_max(linc);
                const float hi = fmaxf(lm, li), lo = fminf(lm, li);
                const float ltot = lo > -INFINITY ? hi + log2_(1.f + exp2_(lo - hi)) : hi;
                delta = fmaxf(floorf(ltot) - 3.f, sig1 - kSigMax);
                mb = exp2_(ltot - delta);
            } else {
                mb = mbn;
            }
            sig1 -= delta;
            const float dsc = exp2_(fminf(-delta, 126.f));
            const bool scaled = tsc != 1.f || eB != 0 || eU != 0 || delta != 0.f;
            float *cwl = sm.cw[w][0];
            if (scaled) {
                if (lane < 32) {
                    cwl[2 * C + lane] = exp2_(fminf(gCp - sm.gl[p][lane] + sig1 + lus, 126.f)) * sm.ks[p][lane];
                    if (WANT_O) cwl[3 * C + lane] = (NORM_Q ? 1.f : sm.kq[p][lane]) * exp2_(lus - (float)eU);
                }
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    if (WANT_O) pc[tt] = cwl[3 * C + 16 * tt + n];
                    c2[tt] = lds_ld<floatx4>(sm, cwb + 4 * (2 * C + 16 * tt + 4 * g));
                }
            }

            // o^T = cw1 Z^T + cw3 (U'^T P^T): lane holds token 16 tt + n, columns 4 g .. 4 g + 3
            if (WANT_O) {
                half8 uf = cat(h4(U2[0]), h4(U2[1]));
                if (eU != 0) {
                    const float sc = ldexpf(1.f, eU);
                    uf = cat(h4(U2[0] * sc), h4(U2[1] * sc));
                }
                const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
                const floatx4 PO[2] = {mfma16(uf, pf0, z4), mfma16(uf, pf1, z4)};
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const int t = 16 * tt + n;
                    float ov[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) ov[j] = zc[tt] * Z2[tt][j] + pc[tt] * PO[tt][j];
                    if (out && t < lc) {
                        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                        typedef __attribute__((address_space(1))) u32x2 gu32x2;
                        gu32x2 *dst = (gu32x2 *)((gchar *)at_tok(G.o, cur.t0 + t, G.ts) + (16 * w + 4 * g) * 2);
                        *dst = u32x2{pack_bf16(ov[0], ov[1]), pack_bf16(ov[2], ov[3])};
                    }
                }
            }
            // W' = 2^{sig1} 2^{g_C - g_s} u_s (S2 units), then S2 <- S2 2^{-delta} + K^ T W'
            U2[0] *= c2[0];
            U2[1] *= c2[1];
            const half8 wfr = cat(h4(U2[0]), h4(U2[1]));
            if (delta != 0.f) {
#pragma unroll
                for (int a = 0; a < 8; ++a) S2[a] *= dsc;
            }
#pragma unroll
            for (int a = 0; a < 8; ++a) S2[a] = mfma16(ktf[a], wfr, S2[a]);
            sigma = sig1;

            if (cur.ne < ne_end && P.emit_after[cur.ne] == cur.t0 + lc)
                store_state2(P.emit_base + (((int64_t)b * P.M + P.emit_slot[cur.ne]) * H + h) * DV * DK, S2, sigma,
                             dvr, L2.scol);
        }
        if (STATE) __builtin_amdgcn_s_setprio(0);
        cur = nx;
        nx = nx2;
        p ^= 1;
        vb ^= 1;
    }
    if (STATE && P.state_dst[r]) store_state2(P.state_dst[r] + (int64_t)h * DV * DK, S2, sigma, dvr, L2.scol);
}

template <bool WANT_O, bool NORM_Q, bool ALIAS>
__global__ __launch_bounds__(NT, 2) void chunked_kernel(const LaunchDesc P)
{
    __shared__ Smem sm;
    const uint32_t sm_lds = (uint32_t)reinterpret_cast<uintptr_t>((lvoid_t *)&sm);
    // work items without outputs (the split prefill's zero-start replays and
    // transition products) take the path that skips the query side entirely
    if (WANT_O && (P.wflags[xcd_remap(blockIdx.x, gridDim.x) / P.H] & kWorkNoOut)) {
        switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
            case 0: wave_main<0, false, NORM_Q, ALIAS>(P, sm, sm_lds); break;
            case 1: wave_main<1, false, NORM_Q, ALIAS>(P, sm, sm_lds); break;
            case 2: wave_main<2, false, NORM_Q, ALIAS>(P, sm, sm_lds); break;
            default: wave_main<3, false, NORM_Q, ALIAS>(P, sm, sm_lds); break;
        }
        return;
    }
    switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
        case 0: wave_main<0, WANT_O, NORM_Q, ALIAS>(P, sm, sm_lds); break;
        case 1: wave_main<1, WANT_O, NORM_Q, ALIAS>(P, sm, sm_lds); break;
        case 2: wave_main<2, WANT_O, NORM_Q, ALIAS>(P, sm, sm_lds); break;
        default: wave_main<3, WANT_O, NORM_Q, ALIAS>(P, sm, sm_lds); break;
    }
}

// Eight waves per workgroup for launches with at most one workgroup per CU:
// waves 0-3 carry the state chain, waves 4-7 the key side (same schedule and
// LDS layout as chunked_kernel), so that the two halves of each phase overlap.
template <bool WANT_O, bool NORM_Q, bool ALIAS>
__global__ __launch_bounds__(2 * NT, 2) void chunked8_kernel(const LaunchDesc P)
{
    __shared__ Smem sm;
    const uint32_t sm_lds = (uint32_t)reinterpret_cast<uintptr_t>((lvoid_t *)&sm);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // (work items without outputs run this path with their stores off; only
    // the four-wave kernel has the path without the query side, for the large
    // launches where the split prefill's side scans matter)
    switch (wv) {
        case 0: wave_main<0, WANT_O, NORM_Q, ALIAS, true>(P, sm, sm_lds); break;
        case 1: wave_main<1, WANT_O, NORM_Q, ALIAS, true>(P, sm, sm_lds); break;
        case 2: wave_main<2, WANT_O, NORM_Q, ALIAS, true>(P, sm, sm_lds); break;
        case 3: wave_main<3, WANT_O, NORM_Q, ALIAS, true>(P, sm, sm_lds); break;
        case 4: wave_main<4, WANT_O, NORM_Q, ALIAS, true>(P, sm, sm_lds); break;
        case 5: wave_main<5, WANT_O, NORM_Q, ALIAS, true>(P, sm, sm_lds); break;
        case 6: wave_main<6, WANT_O, NORM_Q, ALIAS, true>(P, sm, sm_lds); break;
        default: wave_main<7, WANT_O, NORM_Q, ALIAS, true>(P, sm, sm_lds); break;
    }
}

// A group of layers in one launch (identity mixing: layer l + 1 reads layer l's
// outputs as its q = k = v, on the same span).  Each workgroup takes its
// (request, head) through the layers in turn with the four-wave schedule, so
// that results are bit for bit those of one launch per layer; a workgroup that
// finishes a layer starts the next one without waiting for the rest of the
// grid.  Between layers every wave's output stores complete (workgroup-scope
// release, barrier, acquire) before any wave copies them back as the next
// layer's rows: the rows of a (request, head) are written and read by the same
// workgroup, through the same CU's caches and L2 (a device-scope fence, which
// writes back L2, made the launch 15% slower).
template <bool NORM_Q>
__global__ __launch_bounds__(NT, 2) void chunked_group_kernel(const LaunchDesc P, const GroupPtrs gp)
{
    __shared__ Smem sm;
    const uint32_t sm_lds = (uint32_t)reinterpret_cast<uintptr_t>((lvoid_t *)&sm);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int l = 0; l < gp.L; ++l) {
        // constant indices (a dynamic index into the arguments would copy them to scratch)
        GroupLayer lp;
        switch (l) {
            case 0: lp = gp.layer[0]; break;
            case 1: lp = gp.layer[1]; break;
            case 2: lp = gp.layer[2]; break;
            default: lp = gp.layer[kMaxGroupLayers - 1]; break;
        }
        if (l == 0) {
            switch (wv) {
                case 0: wave_main<0, true, NORM_Q, false, false, true>(P, sm, sm_lds, lp); break;
                case 1: wave_main<1, true, NORM_Q, false, false, true>(P, sm, sm_lds, lp); break;
                case 2: wave_main<2, true, NORM_Q, false, false, true>(P, sm, sm_lds, lp); break;
                default: wave_main<3, true, NORM_Q, false, false, true>(P, sm, sm_lds, lp); break;
            }
        } else {
            switch (wv) {
                case 0: wave_main<0, true, NORM_Q, true, false, true>(P, sm, sm_lds, lp); break;
                case 1: wave_main<1, true, NORM_Q, true, false, true>(P, sm, sm_lds, lp); break;
                case 2: wave_main<2, true, NORM_Q, true, false, true>(P, sm, sm_lds, lp); break;
                default: wave_main<3, true, NORM_Q, true, false, true>(P, sm, sm_lds, lp); break;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
}

// Two workgroups of eight waves per (request, head), one per half of d_v
// (dv2_main); grid 2 x pairs, consecutive blocks the two halves of a pair.
// Twelve waves: 0-3 the state side, 4-11 the key side (eight roles).
constexpr int NKV2 = 8;
template <bool WANT_O, bool NORM_Q>
__global__ __launch_bounds__((4 + NKV2) * 64, 3) void chunked_dv2_kernel(const LaunchDesc P)
{
    __shared__ Smem sm;
    const uint32_t sm_lds = (uint32_t)reinterpret_cast<uintptr_t>((lvoid_t *)&sm);
    // (work items without outputs run this path with their stores off)
    switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
        case 0: dv2_main<0, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
        case 1: dv2_main<1, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
        case 2: dv2_main<2, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
        case 3: dv2_main<3, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
        case 4: dv2_main<4, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
        case 5: dv2_main<5, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
        case 6: dv2_main<6, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
        case 7: dv2_main<7, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
        case 8: dv2_main<8, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
        case 9: dv2_main<9, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
        case 10: dv2_main<10, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
        default: dv2_main<11, WANT_O, NORM_Q, NKV2>(P, sm, sm_lds); break;
    }
}

// CUs of the current device, read once per device (0 if the query fails: every
// launch then takes the four-wave kernel).
int cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices && (c = cached[dev].load(std::memory_order_relaxed)) > 0) return c;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 0) return 0;
    if (dev < kMaxDevices) cached[dev].store(c, std::memory_order_relaxed);
    return c;
}

template <bool WANT_O, bool NORM_Q, bool ALIAS>
void launch_variant(const LaunchDesc &d, int nwg, hipStream_t s) {
    if (nwg <= cu_count())
        hipLaunchKernelGGL((chunked8_kernel<WANT_O, NORM_Q, ALIAS>), dim3(nwg), dim3(2 * NT), 0, s, d);
    else
        hipLaunchKernelGGL((chunked_kernel<WANT_O, NORM_Q, ALIAS>), dim3(nwg), dim3(NT), 0, s, d);
}

}  // namespace

hipError_t launch_chunked_group(const LaunchDesc &d, const GroupPtrs &g, hipStream_t s) {
    const int nwg = d.nreq * d.H;
    // only where one launch per layer would run the four-wave kernel on every
    // layer (the results are then the same bits)
    if (g.L < 1 || g.L > kMaxGroupLayers || nwg <= cu_count() || d.o == nullptr) return hipErrorNotSupported;
    if (d.flags & kNormQ) hipLaunchKernelGGL((chunked_group_kernel<true>), dim3(nwg), dim3(NT), 0, s, d, g);
    else hipLaunchKernelGGL((chunked_group_kernel<false>), dim3(nwg), dim3(NT), 0, s, d, g);
    return hipGetLastError();
}

bool chunked_supported(int dk, int dv, Elem e) {
    return dk == DK && dv == DV && e == Elem::BF16;
}

hipError_t launch_chunked(const LaunchDesc &d, int dk, int dv, Elem e, hipStream_t s) {
    if (!chunked_supported(dk, dv, e)) return hipErrorNotSupported;
    const int nwg = d.nreq * d.H;
    if (nwg == 0) return hipSuccess;
    const bool want_o = d.o != nullptr, norm_q = (d.flags & kNormQ) != 0, alias = (d.flags & kAliasQKV) != 0;
    // at most half a workgroup per CU: two eight-wave workgroups per pair, one
    // per half of d_v; one workgroup per CU or fewer: the eight-wave kernel;
    // otherwise two four-wave workgroups share a CU
    if (!alias && 2 * nwg <= cu_count()) {
        const dim3 grid(2 * nwg), block((4 + NKV2) * 64);
        if (want_o && norm_q) hipLaunchKernelGGL((chunked_dv2_kernel<true, true>), grid, block, 0, s, d);
        else if (want_o) hipLaunchKernelGGL((chunked_dv2_kernel<true, false>), grid, block, 0, s, d);
        else if (norm_q) hipLaunchKernelGGL((chunked_dv2_kernel<false, true>), grid, block, 0, s, d);
        else hipLaunchKernelGGL((chunked_dv2_kernel<false, false>), grid, block, 0, s, d);
        return hipGetLastError();
    }
    if (alias) {
        if (want_o && norm_q) launch_variant<true, true, true>(d, nwg, s);
        else if (want_o) launch_variant<true, false, true>(d, nwg, s);
        else if (norm_q) launch_variant<false, true, true>(d, nwg, s);
        else launch_variant<false, false, true>(d, nwg, s);
    } else {
        if (want_o && norm_q) launch_variant<true, true, false>(d, nwg, s);
        else if (want_o) launch_variant<true, false, false>(d, nwg, s);
        else if (norm_q) launch_variant<false, true, false>(d, nwg, s);
        else launch_variant<false, false, false>(d, nwg, s);
    }
    return hipGetLastError();
}

}  // namespace gdn
