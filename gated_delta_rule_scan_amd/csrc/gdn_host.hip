// Host side of libgdnreplay: argument validation, exact integer span logic,
// packing of the per-launch descriptors, and the exported C ABI declared in
// include/gdnreplay.h.  No device memory is allocated and nothing is
// synchronised; every launch is queued on the caller's stream.
//
// Span logic:
//  - tail replay ("Tail-Replay: Escaping the Curse of Linear Attention in
//    Prefix Caching for Hybrid LLMs" §2.1 symbol table and §2.2): k = ceil(r m)
//    in exact integers, positions m - k + 1 .. m, zero start;
//  - resume ("Sparse prefix caching for hybrid and recurrent LLM serving" §3):
//    the deepest checkpoint c_j <= d (none: zero start), positions c_j + 1 .. d;
//  - prefill with emission (same page, §3): positions 1 .. N from zero, the
//    state after each checkpoint position is stored;
//  - the split prefill: the same in three segments per span, joined by the
//    exact split of the Tail-Replay page §2.3 (S_end = S_start P + S^, with
//    the transition product P scanned as v = 0 from the identity);
//  - tail replay with a host-to-device transfer on a second stream (same
//    page, §2.5).
// Apart from the split prefill's caller-provided workspace, no device memory
// beyond the caller's inputs and outputs is used.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gdnreplay.h"
#include "gdn_error.h"
#include "gdn_launch.h"

#define GDN_API extern "C" __attribute__((visibility("default")))

static_assert(gdn::kMaxEmitPerLaunch >= GDN_MAX_CHECKPOINTS,
              "one request's emissions must fit one launch");

namespace {

thread_local std::string g_last_error;

gdn_status vfail(gdn_status st, const char *fmt, va_list ap) {
    char buf[512];
    vsnprintf(buf, sizeof(buf), fmt, ap);
    g_last_error = buf;
    return st;
}

gdn_status fail(gdn_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    const gdn_status r = vfail(st, fmt, ap);
    va_end(ap);
    return r;
}

bool valid_width(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

constexpr uint32_t kKnownFlags =
    GDN_NORMALIZE_K | GDN_NORMALIZE_Q | GDN_KERNEL_RECURRENT | GDN_KERNEL_CHUNKED;

// One work item: scan `len` tokens of request b starting at packed row `row0`,
// from the state at `init_off` (-1: zero), emitting at span-relative counts,
// final state to dst ([H][d_v][d_k], NULL: not stored); wflags: gdn::kWork*.
struct Work {
    int32_t b;
    int64_t row0;
    int64_t len;
    int64_t init_off;
    std::vector<std::pair<int32_t, int32_t>> emits;  // (count after, slot)
    float *dst = nullptr;
    int32_t wflags = 0;
};

gdn_status check_shape(const gdn_shape *s) {
    if (!s) return fail(GDN_ERR_INVALID_ARGUMENT, "shape is NULL");
    if (s->B < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "B = %d < 0", s->B);
    if (s->H < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "H = %d < 1", s->H);
    if (!valid_width(s->dk) || !valid_width(s->dv))
        return fail(GDN_ERR_UNSUPPORTED, "d_k = %d, d_v = %d: each must be 16, 32, 64 or 128",
                    s->dk, s->dv);
    if (s->dtype != GDN_DTYPE_F32 && s->dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_INVALID_ARGUMENT, "unknown dtype %d", s->dtype);
    if (s->flags & ~kKnownFlags)
        return fail(GDN_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", s->flags & ~kKnownFlags);
    if ((s->flags & GDN_KERNEL_RECURRENT) && (s->flags & GDN_KERNEL_CHUNKED))
        return fail(GDN_ERR_INVALID_ARGUMENT, "GDN_KERNEL_RECURRENT and GDN_KERNEL_CHUNKED both set");
    return GDN_OK;
}

gdn_status check_rows(const gdn_shape *s, const int64_t *off, const int64_t *first) {
    if (!off) return fail(GDN_ERR_INVALID_ARGUMENT, "h_tok_offset is NULL");
    if (off[0] < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "h_tok_offset[0] = %lld < 0", (long long)off[0]);
    for (int32_t b = 0; b < s->B; ++b) {
        if (off[b + 1] < off[b])
            return fail(GDN_ERR_INVALID_ARGUMENT, "h_tok_offset decreases at request %d", b);
        if (first && first[b] < 1)
            return fail(GDN_ERR_INVALID_ARGUMENT, "h_first_pos[%d] = %lld < 1", b, (long long)first[b]);
    }
    const int64_t rows = off[s->B];
    const int64_t wmax = s->dk > s->dv ? s->dk : s->dv;
    if (rows > (INT64_MAX / 4) / ((int64_t)s->H * wmax))
        return fail(GDN_ERR_INVALID_ARGUMENT, "too many rows (%lld)", (long long)rows);
    return GDN_OK;
}

// The span [p0, p0 + len) must lie inside the stored rows of request b.
gdn_status span_to_rows(int32_t b, const int64_t *off, const int64_t *first, int64_t p0,
                        int64_t len, int64_t *row0) {
    const int64_t f = first ? first[b] : 1;
    const int64_t n = off[b + 1] - off[b];
    *row0 = off[b] + (p0 - f);
    if (len == 0) {
        *row0 = off[b];
        return GDN_OK;
    }
    if (p0 < f || p0 + len - 1 > f + n - 1)
        return fail(GDN_ERR_INVALID_ARGUMENT,
                    "request %d: span positions %lld..%lld are not stored (rows hold %lld..%lld)",
                    b, (long long)p0, (long long)(p0 + len - 1), (long long)f, (long long)(f + n - 1));
    if (len > INT32_MAX)
        return fail(GDN_ERR_UNSUPPORTED, "request %d: span of %lld tokens exceeds 2^31 - 1", b,
                    (long long)len);
    return GDN_OK;
}

gdn_status check_positions(const int64_t *pos, int32_t B, int32_t M) {
    if (M < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "M = %d < 0", M);
    if (M > GDN_MAX_CHECKPOINTS)
        return fail(GDN_ERR_UNSUPPORTED, "M = %d exceeds %d checkpoints per request", M,
                    GDN_MAX_CHECKPOINTS);
    if (M > 0 && B > 0 && !pos) return fail(GDN_ERR_INVALID_ARGUMENT, "h_ckpt_pos is NULL");
    for (int32_t b = 0; b < B; ++b)
        for (int32_t i = 0; i < M; ++i) {
            const int64_t c = pos[(int64_t)b * M + i];
            if (c < 1)
                return fail(GDN_ERR_INVALID_ARGUMENT, "request %d: checkpoint %d at %lld < 1", b, i,
                            (long long)c);
            if (i > 0 && c <= pos[(int64_t)b * M + i - 1])
                return fail(GDN_ERR_INVALID_ARGUMENT,
                            "request %d: checkpoint positions not strictly increasing at %d", b, i);
        }
    return GDN_OK;
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
    const char *pa = static_cast<const char *>(a);
    const char *pb = static_cast<const char *>(b);
    return pa < pb + nb && pb < pa + na;
}

// 0: per-token kernel, 1: chunked kernel, -1: GDN_KERNEL_CHUNKED cannot be honoured.
// The chunked kernel needs unit keys: its fp16 operand ranges rely on them.
int32_t kernel_choice(const gdn_shape *s) {
    const gdn::Elem elem = s->dtype == GDN_DTYPE_F32 ? gdn::Elem::F32 : gdn::Elem::BF16;
    const bool has_chunked =
        gdn::chunked_supported(s->dk, s->dv, elem) && (s->flags & GDN_NORMALIZE_K);
    if ((s->flags & GDN_KERNEL_CHUNKED) && !has_chunked) return -1;
    return (has_chunked && !(s->flags & GDN_KERNEL_RECURRENT)) ? 1 : 0;
}

// Final states of request b go to state_out + b H d_v d_k.
gdn_status set_state_out(std::vector<Work> &work, float *state_out, const gdn_shape *s) {
    if (!state_out && !work.empty()) return fail(GDN_ERR_INVALID_ARGUMENT, "state_out is NULL");
    const int64_t slot = (int64_t)s->H * s->dv * s->dk;
    for (Work &w : work) w.dst = state_out + (int64_t)w.b * slot;
    return GDN_OK;
}

bool misaligned(const void *p, uintptr_t a) { return p && (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// A validated call: the kernel to run and the launch descriptor's common part.
struct Plan {
    bool chunked = false;
    gdn::Elem elem = gdn::Elem::BF16;
    gdn::LaunchDesc d;
};

// Validate pointers and alignment and pick the kernel; nothing is queued.
gdn_status validate(const gdn_shape *s, const void *q, const void *k, const void *v,
                    const void *alpha, const void *beta, void *o,
                    const float *init_base, float *emit_base, int32_t M,
                    const std::vector<Work> &work, Plan *plan) {
    bool any_tokens = false;
    for (const Work &w : work) any_tokens |= w.len > 0;
    if (any_tokens) {
        if (!k || !v || !alpha || !beta)
            return fail(GDN_ERR_INVALID_ARGUMENT, "k, v, alpha and beta must be non-NULL");
        if (o && !q) return fail(GDN_ERR_INVALID_ARGUMENT, "o is set but q is NULL");
    }
    // inputs at their element size; states are read and written as float4
    const uintptr_t esz = s->dtype == GDN_DTYPE_F32 ? 4 : 2;
    if (misaligned(q, esz) || misaligned(k, esz) || misaligned(v, esz) || misaligned(alpha, esz) ||
        misaligned(beta, esz) || misaligned(o, esz))
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, alpha, beta and o must be aligned to their element size");
    if (misaligned(init_base, 16) || misaligned(emit_base, 16))
        return fail(GDN_ERR_INVALID_ARGUMENT, "the checkpoint store must be 16-byte aligned");
    for (const Work &w : work)
        if (misaligned(w.dst, 16)) return fail(GDN_ERR_INVALID_ARGUMENT, "state_out must be 16-byte aligned");
    // the chunked kernel copies 16-byte pieces of q, k, v rows and stores whole o rows
    const bool rows16 = !misaligned(q, 16) && !misaligned(k, 16) && !misaligned(v, 16) && !misaligned(o, 16);
    int32_t kern = kernel_choice(s);
    if (kern == 1 && !rows16) {
        if (s->flags & GDN_KERNEL_CHUNKED)
            return fail(GDN_ERR_UNSUPPORTED, "GDN_KERNEL_CHUNKED: q, k, v and o must be 16-byte aligned");
        kern = 0;
    }
    if (kern < 0)
        return fail(GDN_ERR_UNSUPPORTED,
                    "GDN_KERNEL_CHUNKED: no chunked kernel for d_k = %d, d_v = %d, dtype %d, flags 0x%x "
                    "(it needs bf16, d_k = d_v = 128 and GDN_NORMALIZE_K)",
                    s->dk, s->dv, s->dtype, s->flags);
    // the kernels write o and the states while they read the inputs: the
    // span rows of q, k, v, alpha and beta must not share memory with either
    if (any_tokens) {
        int64_t r0 = INT64_MAX, r1 = INT64_MIN;
        for (const Work &w : work)
            if (w.len > 0) {
                r0 = std::min(r0, w.row0);
                r1 = std::max(r1, w.row0 + w.len);
            }
        const size_t row = (size_t)s->H * esz;  // bytes of one row per unit of width
        auto span_of = [&](const void *p, int64_t width) {
            return std::make_pair(p ? static_cast<const char *>(p) + (size_t)r0 * row * (size_t)width : nullptr,
                                  (size_t)(r1 - r0) * row * (size_t)width);
        };
        const std::pair<const char *, size_t> in[5] = {span_of(q, s->dk), span_of(k, s->dk), span_of(v, s->dv),
                                                       span_of(alpha, 1), span_of(beta, 1)};
        const auto out = span_of(o, s->dv);
        const size_t slot = (size_t)s->H * s->dv * s->dk * sizeof(float);
        int32_t nb = 0;  // requests covered by the emission store
        for (const Work &w : work) nb = std::max(nb, w.b + 1);
        for (const auto &e : in) {
            if (!e.first) continue;
            if (out.first && ranges_overlap(out.first, out.second, e.first, e.second))
                return fail(GDN_ERR_INVALID_ARGUMENT, "o overlaps q, k, v, alpha or beta on the span rows");
            for (const Work &w : work)
                if (w.dst && ranges_overlap(w.dst, slot, e.first, e.second))
                    return fail(GDN_ERR_INVALID_ARGUMENT, "a state buffer overlaps q, k, v, alpha or beta");
            if (emit_base && M > 0 && ranges_overlap(emit_base, (size_t)nb * M * slot, e.first, e.second))
                return fail(GDN_ERR_INVALID_ARGUMENT, "ckpt_states overlaps q, k, v, alpha or beta");
        }
    }
    plan->elem = s->dtype == GDN_DTYPE_F32 ? gdn::Elem::F32 : gdn::Elem::BF16;
    plan->chunked = kern == 1;

    gdn::LaunchDesc &d = plan->d;
    std::memset(&d, 0, sizeof(d));
    d.q = q;
    d.k = k;
    d.v = v;
    d.alpha = alpha;
    d.beta = beta;
    d.o = o;
    d.init_base = init_base;
    d.emit_base = emit_base;
    d.H = s->H;
    d.flags = (int32_t)(s->flags & (GDN_NORMALIZE_K | GDN_NORMALIZE_Q));
    // one tensor for q, k and v (a layer fed its predecessor's outputs): the
    // chunked kernel then reads each row once
    if (plan->chunked && k && k == v && s->dk == s->dv && (!o || q == k)) d.flags |= gdn::kAliasQKV;
    d.M = M;
    return GDN_OK;
}

// Queue the launches of a validated call (several when the work items or
// their emissions exceed one descriptor).
// Packs the requests from work[i] on into d, as many as one launch takes (d.nreq);
// returns the index of the first request left for the next launch.
size_t pack_launch(gdn::LaunchDesc &d, const std::vector<Work> &work, size_t i) {
    int nreq = 0, nemit = 0;
    d.emit_begin[0] = 0;
    while (i < work.size() && nreq < gdn::kMaxReqPerLaunch &&
           nemit + (int)work[i].emits.size() <= gdn::kMaxEmitPerLaunch) {
        const Work &w = work[i];
        d.row0[nreq] = w.row0;
        d.init_off[nreq] = w.init_off;
        d.len[nreq] = (int32_t)w.len;
        d.req[nreq] = w.b;
        d.state_dst[nreq] = w.dst;
        d.wflags[nreq] = w.wflags;
        for (const auto &e : w.emits) {
            d.emit_after[nemit] = e.first;
            d.emit_slot[nemit] = e.second;
            ++nemit;
        }
        d.emit_begin[nreq + 1] = nemit;
        ++nreq;
        ++i;
    }
    d.nreq = nreq;
    return i;
}

hipError_t launch_one(const gdn_shape *s, const Plan &plan, hipStream_t stream) {
    return plan.chunked ? gdn::launch_chunked(plan.d, s->dk, s->dv, plan.elem, stream)
                        : gdn::launch_recurrent(plan.d, s->dk, s->dv, plan.elem, stream);
}

gdn_status launch(const gdn_shape *s, Plan &plan, const std::vector<Work> &work, hipStream_t stream) {
    size_t i = 0;
    while (i < work.size()) {
        i = pack_launch(plan.d, work, i);
        if (plan.d.nreq == 0)  // cannot happen: one request never exceeds the emission budget
            return fail(GDN_ERR_UNSUPPORTED, "emission list does not fit one launch");
        const hipError_t err = launch_one(s, plan, stream);
        if (err != hipSuccess)
            return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    }
    return GDN_OK;
}

// Validate, then queue the launches.
gdn_status run(const gdn_shape *s, const void *q, const void *k, const void *v,
               const void *alpha, const void *beta, void *o,
               const float *init_base, float *emit_base, int32_t M,
               const std::vector<Work> &work, hipStream_t stream) {
    Plan plan;
    const gdn_status st = validate(s, q, k, v, alpha, beta, o, init_base, emit_base, M, work, &plan);
    if (st != GDN_OK) return st;
    return launch(s, plan, work, stream);
}

int64_t tail_len_exact(int64_t m, int64_t r_num, int64_t r_den) {
    if (m < 0 || r_num < 0 || r_den <= 0) return -1;
    const __int128 num = (__int128)m * r_num;
    __int128 k = (num + r_den - 1) / r_den;  // ceiling of a non-negative ratio
    if (k > m) k = m;
    return (int64_t)k;
}

int32_t select_exact(const int64_t *pos, int32_t M, int64_t depth) {
    int32_t j = 0;
    for (int32_t i = 0; i < M; ++i)
        if (pos[i] <= depth) j = i + 1;
    return j;
}

}  // namespace

gdn_status gdn::host_fail(gdn_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    const gdn_status r = vfail(st, fmt, ap);
    va_end(ap);
    return r;
}

GDN_API const char *gdn_version(void) { return "libgdnreplay 0.1.0 gfx950"; }

GDN_API const char *gdn_last_error(void) { return g_last_error.c_str(); }

GDN_API int32_t gdn_kernel_for(const gdn_shape *shape) {
    if (check_shape(shape) != GDN_OK) return -1;
    return kernel_choice(shape);
}

GDN_API int64_t gdn_tail_len(int64_t m, int64_t r_num, int64_t r_den) {
    return tail_len_exact(m, r_num, r_den);
}

GDN_API int32_t gdn_select_checkpoint(const int64_t *pos, int32_t M, int64_t depth) {
    if (M < 0 || depth < 0 || (M > 0 && !pos)) return -1;
    for (int32_t i = 0; i < M; ++i)
        if (pos[i] < 1 || (i > 0 && pos[i] <= pos[i - 1])) return -1;
    return select_exact(pos, M, depth);
}

namespace {

// Validation and span logic of a tail replay; fills work and ks (B entries).
gdn_status prepare_tail(const gdn_shape *shape, const int64_t *h_tok_offset, const int64_t *h_first_pos,
                        const int64_t *h_m, int64_t r_num, int64_t r_den, std::vector<Work> &work,
                        std::vector<int64_t> &ks) {
    gdn_status st = check_shape(shape);
    if (st != GDN_OK) return st;
    if (shape->B == 0) return GDN_OK;
    if ((st = check_rows(shape, h_tok_offset, h_first_pos)) != GDN_OK) return st;
    if (!h_m) return fail(GDN_ERR_INVALID_ARGUMENT, "h_m is NULL");
    if (r_num < 0 || r_den <= 0)
        return fail(GDN_ERR_INVALID_ARGUMENT, "replay ratio %lld/%lld invalid", (long long)r_num,
                    (long long)r_den);
    work.assign(shape->B, Work{});
    ks.assign(shape->B, 0);
    for (int32_t b = 0; b < shape->B; ++b) {
        if (h_m[b] < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "h_m[%d] < 0", b);
        const int64_t kb = tail_len_exact(h_m[b], r_num, r_den);
        ks[b] = kb;
        Work &w = work[b];
        w.b = b;
        w.len = kb;
        w.init_off = -1;
        if ((st = span_to_rows(b, h_tok_offset, h_first_pos, h_m[b] - kb + 1, kb, &w.row0)) != GDN_OK)
            return st;
    }
    return GDN_OK;
}

}  // namespace

GDN_API gdn_status gdn_tail_replay(const gdn_shape *shape, const void *q, const void *k,
                                   const void *v, const void *alpha, const void *beta,
                                   const int64_t *h_tok_offset, const int64_t *h_first_pos,
                                   const int64_t *h_m, int64_t r_num, int64_t r_den,
                                   float *state_out, void *o, int64_t *h_k_out,
                                   hipStream_t stream) {
    g_last_error.clear();
    std::vector<Work> work;
    std::vector<int64_t> ks;
    gdn_status st = prepare_tail(shape, h_tok_offset, h_first_pos, h_m, r_num, r_den, work, ks);
    if (st != GDN_OK || shape->B == 0) return st;
    if ((st = set_state_out(work, state_out, shape)) != GDN_OK) return st;
    st = run(shape, q, k, v, alpha, beta, o, nullptr, nullptr, 0, work, stream);
    if (st == GDN_OK && h_k_out)
        for (int32_t b = 0; b < shape->B; ++b) h_k_out[b] = ks[b];
    return st;
}

GDN_API gdn_status gdn_tail_replay_group(const gdn_shape *shape, int32_t L, const void *q, const void *k,
                                         const void *v, const void *const *alpha, const void *const *beta,
                                         const int64_t *h_tok_offset, const int64_t *h_first_pos,
                                         const int64_t *h_m, int64_t r_num, int64_t r_den, float *state_out,
                                         void *o, int64_t *h_k_out, hipStream_t stream) {
    g_last_error.clear();
    if (L < 1 || L > gdn::kMaxGroupLayers)
        return fail(GDN_ERR_INVALID_ARGUMENT, "L = %d layers, 1..%d supported", L, gdn::kMaxGroupLayers);
    if (!alpha || !beta) return fail(GDN_ERR_INVALID_ARGUMENT, "alpha and beta (host arrays of L pointers) are NULL");
    std::vector<Work> work;
    std::vector<int64_t> ks;
    gdn_status st = prepare_tail(shape, h_tok_offset, h_first_pos, h_m, r_num, r_den, work, ks);
    if (st != GDN_OK || shape->B == 0) return st;
    if (shape->dk != shape->dv)
        return fail(GDN_ERR_UNSUPPORTED, "a group feeds each layer's outputs to the next as q = k = v: d_k = d_v "
                                         "needed (got %d, %d)", shape->dk, shape->dv);
    if (!o) return fail(GDN_ERR_INVALID_ARGUMENT, "o is NULL (each layer's outputs are the next layer's inputs)");
    if (!state_out) return fail(GDN_ERR_INVALID_ARGUMENT, "state_out is NULL");
    const int64_t rows = h_tok_offset[shape->B];
    const size_t esz = shape->dtype == GDN_DTYPE_F32 ? 4 : 2;
    const size_t oslab = (size_t)rows * shape->H * shape->dv * esz;                   // bytes per layer
    const int64_t sslab = (int64_t)shape->B * shape->H * shape->dv * shape->dk;      // floats per layer
    if (ranges_overlap(o, (size_t)L * oslab, state_out, (size_t)L * sslab * sizeof(float)))
        return fail(GDN_ERR_INVALID_ARGUMENT, "o and state_out overlap");
    auto o_of = [&](int32_t l) { return static_cast<void *>(static_cast<char *>(o) + (size_t)l * oslab); };
    // layer l: its own state slab; q = k = v = the outputs of layer l - 1
    std::vector<Plan> plans((size_t)L);
    std::vector<std::vector<Work>> lw((size_t)L, work);
    for (int32_t l = 0; l < L; ++l) {
        if ((st = set_state_out(lw[(size_t)l], state_out + (int64_t)l * sslab, shape)) != GDN_OK) return st;
        const void *ql = l ? o_of(l - 1) : q, *kl = l ? o_of(l - 1) : k, *vl = l ? o_of(l - 1) : v;
        if ((st = validate(shape, ql, kl, vl, alpha[l], beta[l], o_of(l), nullptr, nullptr, 0, lw[(size_t)l],
                           &plans[(size_t)l])) != GDN_OK)
            return st;
    }
    bool all_chunked = true;
    for (const Plan &pl : plans) all_chunked = all_chunked && pl.chunked;
    size_t i = 0;
    while (i < work.size()) {
        size_t next = i;
        for (int32_t l = 0; l < L; ++l) next = pack_launch(plans[(size_t)l].d, lw[(size_t)l], i);
        i = next;
        // one launch for every layer of these requests where it gives the same
        // bits as one launch per layer; otherwise one launch per layer
        hipError_t err = hipErrorNotSupported;
        if (all_chunked) {
            gdn::GroupPtrs g{};
            g.L = L;
            for (int32_t l = 0; l < L; ++l) {
                const gdn::LaunchDesc &dl = plans[(size_t)l].d;
                g.layer[l] = gdn::GroupLayer{dl.q, dl.k, dl.v, dl.alpha, dl.beta, dl.o, (int64_t)l * sslab};
            }
            err = gdn::launch_chunked_group(plans[0].d, g, stream);
        }
        if (err == hipErrorNotSupported) {
            for (int32_t l = 0; l < L && (err = launch_one(shape, plans[(size_t)l], stream)) == hipSuccess; ++l) {
            }
        }
        if (err != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    }
    if (h_k_out)
        for (int32_t b = 0; b < shape->B; ++b) h_k_out[b] = ks[b];
    return GDN_OK;
}

GDN_API gdn_status gdn_tail_replay_with_h2d(const gdn_shape *shape, const void *q, const void *k,
                                            const void *v, const void *alpha, const void *beta,
                                            const int64_t *h_tok_offset, const int64_t *h_first_pos,
                                            const int64_t *h_m, int64_t r_num, int64_t r_den,
                                            float *state_out, void *o, int64_t *h_k_out,
                                            void *kv_dst, const void *kv_src, size_t kv_bytes,
                                            hipStream_t stream, hipStream_t copy_stream,
                                            hipEvent_t copy_done) {
    g_last_error.clear();
    std::vector<Work> work;
    std::vector<int64_t> ks;
    gdn_status st = prepare_tail(shape, h_tok_offset, h_first_pos, h_m, r_num, r_den, work, ks);
    if (st != GDN_OK) return st;
    if ((st = set_state_out(work, state_out, shape)) != GDN_OK) return st;
    if (kv_bytes > 0 && (!kv_dst || !kv_src))
        return fail(GDN_ERR_INVALID_ARGUMENT, "kv_dst or kv_src is NULL with kv_bytes = %zu", kv_bytes);
    if (!copy_done) return fail(GDN_ERR_INVALID_ARGUMENT, "copy_done is NULL");
    // every argument of the replay is checked before anything is queued
    Plan plan;
    if (shape->B > 0 &&
        (st = validate(shape, q, k, v, alpha, beta, o, nullptr, nullptr, 0, work, &plan)) != GDN_OK)
        return st;
    // the transfer goes first, so that the copy engine starts while the replay is queued
    hipError_t e = hipSuccess;
    if (kv_bytes > 0) e = hipMemcpyAsync(kv_dst, kv_src, kv_bytes, hipMemcpyHostToDevice, copy_stream);
    if (e == hipSuccess) e = hipEventRecord(copy_done, copy_stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "transfer: %s", hipGetErrorString(e));
    if (shape->B > 0 && (st = launch(shape, plan, work, stream)) != GDN_OK) return st;
    // work queued on `stream` after this call sees both the replayed states and the transfer
    e = hipStreamWaitEvent(stream, copy_done, 0);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "join: %s", hipGetErrorString(e));
    if (h_k_out)
        for (int32_t b = 0; b < shape->B; ++b) h_k_out[b] = ks[b];
    return GDN_OK;
}

GDN_API gdn_status gdn_resume(const gdn_shape *shape, const void *q, const void *k,
                              const void *v, const void *alpha, const void *beta,
                              const int64_t *h_tok_offset, const int64_t *h_first_pos,
                              const int64_t *h_ckpt_pos, int32_t M, const float *ckpt_states,
                              const int64_t *h_depth, float *state_out, void *o,
                              int32_t *h_j_out, hipStream_t stream) {
    g_last_error.clear();
    gdn_status st = check_shape(shape);
    if (st != GDN_OK) return st;
    if (shape->B == 0) return GDN_OK;
    if ((st = check_rows(shape, h_tok_offset, h_first_pos)) != GDN_OK) return st;
    if ((st = check_positions(h_ckpt_pos, shape->B, M)) != GDN_OK) return st;
    if (!h_depth) return fail(GDN_ERR_INVALID_ARGUMENT, "h_depth is NULL");
    if (!state_out) return fail(GDN_ERR_INVALID_ARGUMENT, "state_out is NULL");
    const int64_t slot = (int64_t)shape->H * shape->dv * shape->dk;  // floats per (b, slot)
    std::vector<Work> work(shape->B);
    std::vector<int32_t> js(shape->B);
    for (int32_t b = 0; b < shape->B; ++b) {
        const int64_t dpt = h_depth[b];
        if (dpt < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "h_depth[%d] < 0", b);
        const int32_t j = select_exact(h_ckpt_pos + (int64_t)b * M, M, dpt);
        js[b] = j;
        const int64_t c = j > 0 ? h_ckpt_pos[(int64_t)b * M + j - 1] : 0;
        Work &w = work[b];
        w.b = b;
        w.len = dpt - c;
        w.init_off = j > 0 ? ((int64_t)b * M + (j - 1)) * slot : -1;
        if (j > 0 && !ckpt_states)
            return fail(GDN_ERR_INVALID_ARGUMENT, "request %d selects checkpoint %d but ckpt_states is NULL", b, j);
        if ((st = span_to_rows(b, h_tok_offset, h_first_pos, c + 1, w.len, &w.row0)) != GDN_OK)
            return st;
    }
    // state_out may coincide with a request's own selected slot; any other
    // overlap with a slot that is read would race.
    if (ckpt_states) {
        const size_t sb = (size_t)slot * sizeof(float);
        for (int32_t b = 0; b < shape->B; ++b) {
            const float *out_b = state_out + (int64_t)b * slot;
            for (int32_t b2 = 0; b2 < shape->B; ++b2) {
                if (work[b2].init_off < 0) continue;
                const float *in_b2 = ckpt_states + work[b2].init_off;
                if (ranges_overlap(out_b, sb, in_b2, sb) && !(b == b2 && out_b == in_b2))
                    return fail(GDN_ERR_INVALID_ARGUMENT,
                                "state_out of request %d overlaps the checkpoint read by request %d", b, b2);
            }
        }
    }
    if ((st = set_state_out(work, state_out, shape)) != GDN_OK) return st;
    st = run(shape, q, k, v, alpha, beta, o, ckpt_states, nullptr, M, work, stream);
    if (st == GDN_OK && h_j_out)
        for (int32_t b = 0; b < shape->B; ++b) h_j_out[b] = js[b];
    return st;
}

namespace {

// Validation and span logic of a prefill: one work per request over 1..N_b.
gdn_status prepare_prefill(const gdn_shape *shape, const int64_t *h_tok_offset, const int64_t *h_first_pos,
                           const int64_t *h_ckpt_pos, int32_t M, float *ckpt_states, float *state_out,
                           std::vector<Work> &work) {
    gdn_status st = check_shape(shape);
    if (st != GDN_OK) return st;
    if (shape->B == 0) return GDN_OK;
    if ((st = check_rows(shape, h_tok_offset, h_first_pos)) != GDN_OK) return st;
    if ((st = check_positions(h_ckpt_pos, shape->B, M)) != GDN_OK) return st;
    if (M > 0 && !ckpt_states) return fail(GDN_ERR_INVALID_ARGUMENT, "ckpt_states is NULL");
    if (!state_out) return fail(GDN_ERR_INVALID_ARGUMENT, "state_out is NULL");
    const int64_t slot = (int64_t)shape->H * shape->dv * shape->dk;
    if (M > 0 && ranges_overlap(state_out, (size_t)shape->B * slot * sizeof(float), ckpt_states,
                                (size_t)shape->B * M * slot * sizeof(float)))
        return fail(GDN_ERR_INVALID_ARGUMENT, "state_out overlaps ckpt_states");
    work.assign(shape->B, Work{});
    for (int32_t b = 0; b < shape->B; ++b) {
        if (h_first_pos && h_first_pos[b] != 1)
            return fail(GDN_ERR_INVALID_ARGUMENT, "prefill needs the whole prefix: h_first_pos[%d] = %lld",
                        b, (long long)h_first_pos[b]);
        const int64_t n = h_tok_offset[b + 1] - h_tok_offset[b];
        Work &w = work[b];
        w.b = b;
        w.len = n;
        w.init_off = -1;
        if ((st = span_to_rows(b, h_tok_offset, nullptr, 1, n, &w.row0)) != GDN_OK) return st;
        for (int32_t i = 0; i < M; ++i) {
            const int64_t c = h_ckpt_pos[(int64_t)b * M + i];
            if (c > n)
                return fail(GDN_ERR_INVALID_ARGUMENT, "request %d: checkpoint %lld beyond N = %lld", b,
                            (long long)c, (long long)n);
            w.emits.emplace_back((int32_t)c, i);
        }
    }
    return GDN_OK;
}

// Spans shorter than this run in one pass in the split prefill.
constexpr int64_t kSplitMinTokens = 768;

}  // namespace

GDN_API gdn_status gdn_prefill_emit_checkpoints(const gdn_shape *shape, const void *q,
                                                const void *k, const void *v,
                                                const void *alpha, const void *beta,
                                                const int64_t *h_tok_offset,
                                                const int64_t *h_first_pos,
                                                const int64_t *h_ckpt_pos, int32_t M,
                                                float *ckpt_states, float *state_out, void *o,
                                                hipStream_t stream) {
    g_last_error.clear();
    std::vector<Work> work;
    gdn_status st = prepare_prefill(shape, h_tok_offset, h_first_pos, h_ckpt_pos, M, ckpt_states, state_out, work);
    if (st != GDN_OK || shape->B == 0) return st;
    if ((st = set_state_out(work, state_out, shape)) != GDN_OK) return st;
    return run(shape, q, k, v, alpha, beta, o, nullptr, ckpt_states, M, work, stream);
}

GDN_API size_t gdn_prefill_split_workspace_bytes(const gdn_shape *shape) {
    if (!shape || shape->B < 0 || shape->H < 1 || shape->dk < 1 || shape->dv < 1) return 0;
    return (size_t)4 * shape->B * shape->H * shape->dv * shape->dk * sizeof(float);
}

namespace {

// The split prefill on a caller's workspace (workspace_bytes long).
gdn_status split_prefill(const gdn_shape *shape, const void *q, const void *k, const void *v,
                         const void *alpha, const void *beta, const int64_t *h_tok_offset,
                         const int64_t *h_first_pos, const int64_t *h_ckpt_pos, int32_t M,
                         float *ckpt_states, float *state_out, void *o, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    std::vector<Work> whole;
    gdn_status st = prepare_prefill(shape, h_tok_offset, h_first_pos, h_ckpt_pos, M, ckpt_states, state_out, whole);
    if (st != GDN_OK || shape->B == 0) return st;
    if (shape->dk != shape->dv)
        return fail(GDN_ERR_UNSUPPORTED, "the split prefill needs d_k = d_v (got %d, %d)", shape->dk, shape->dv);
    const size_t need = gdn_prefill_split_workspace_bytes(shape);
    if (!workspace || workspace_bytes < need)
        return fail(GDN_ERR_INVALID_ARGUMENT, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (misaligned(workspace, 16)) return fail(GDN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    const int64_t slot = (int64_t)shape->H * shape->dv * shape->dk;
    if (ranges_overlap(workspace, need, state_out, (size_t)shape->B * slot * sizeof(float)) ||
        (M > 0 && ranges_overlap(workspace, need, ckpt_states, (size_t)shape->B * M * slot * sizeof(float))))
        return fail(GDN_ERR_INVALID_ARGUMENT, "workspace overlaps state_out or ckpt_states");
    // workspace [4][B][H][d][d]: end of segment 0, zero-start replay and transition
    // product of segment 1, start of segment 2
    float *ws = static_cast<float *>(workspace);
    const int64_t kind = (int64_t)shape->B * slot;
    auto ws_off = [&](int which, int32_t b) { return (int64_t)which * kind + (int64_t)b * slot; };

    std::vector<Work> first, second;  // launches before and after the combine
    bool any_split = false;
    for (Work &w : whole) {
        const int32_t b = w.b;
        const int64_t n = w.len;
        float *out_b = state_out + (int64_t)b * slot;
        const int64_t s1 = (n / 3) & ~(int64_t)31, s2 = (2 * n / 3) & ~(int64_t)31;
        if (n < kSplitMinTokens || s1 <= 0 || s2 <= s1 || s2 >= n) {
            w.dst = out_b;  // short span: one pass
            first.push_back(std::move(w));
            continue;
        }
        any_split = true;
        auto segment = [&](int64_t a0, int64_t len) {
            Work x;
            x.b = b;
            x.row0 = w.row0 + a0;
            x.len = len;
            x.init_off = -1;
            for (const auto &e : w.emits)
                if (e.first > a0 && e.first <= a0 + len) x.emits.emplace_back((int32_t)(e.first - a0), e.second);
            return x;
        };
        Work seg0 = segment(0, s1);
        seg0.dst = ws + ws_off(0, b);
        Work hat1 = segment(s1, s2 - s1);
        hat1.emits.clear();
        hat1.wflags = gdn::kWorkNoOut;
        hat1.dst = ws + ws_off(1, b);
        Work prod1 = hat1;
        prod1.wflags = gdn::kWorkNoOut | gdn::kWorkZeroV | gdn::kWorkIdentity;
        prod1.dst = ws + ws_off(2, b);
        Work seg1 = segment(s1, s2 - s1);
        seg1.init_off = ws_off(0, b);
        seg1.dst = nullptr;
        Work seg2 = segment(s2, n - s2);
        seg2.init_off = ws_off(3, b);
        seg2.dst = out_b;
        first.push_back(std::move(seg0));
        first.push_back(std::move(hat1));
        first.push_back(std::move(prod1));
        second.push_back(std::move(seg1));
        second.push_back(std::move(seg2));
    }
    if ((st = run(shape, q, k, v, alpha, beta, o, nullptr, ckpt_states, M, first, stream)) != GDN_OK) return st;
    if (!any_split) return GDN_OK;
    // start of segment 2 = (end of segment 0) P_1 + S^_1, for every request (the
    // slots of unsplit requests are not read afterwards)
    const hipError_t e = gdn::launch_affine_combine(ws + ws_off(0, 0), ws + ws_off(2, 0), ws + ws_off(1, 0),
                                                    ws + ws_off(3, 0), (int64_t)shape->B * shape->H, shape->dk,
                                                    stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "combine launch failed: %s", hipGetErrorString(e));
    return run(shape, q, k, v, alpha, beta, o, ws, ckpt_states, M, second, stream);
}

// Fixed scratch of the allocation-free split prefill: one array per GPU, in the
// library's code object (held until the process ends).  In host code `scratch`
// names a host-side stand-in, never the device memory: the device address is
// taken per device with hipGetSymbolAddress and only that address is used.
__device__ __align__(256) float scratch[GDN_SPLIT_SCRATCH_BYTES / sizeof(float)];

std::mutex g_scratch_mu;
std::vector<float *> g_scratch_ptr;  // device address of `scratch`, per device (NULL: not taken yet)

// Device address of this device's scratch array, taken once per device with the
// device current.
gdn_status scratch_for_current_device(float **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
    if (!g_scratch_ptr[(size_t)dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[(size_t)dev] = static_cast<float *>(ptr);
    }
    *out = g_scratch_ptr[(size_t)dev];
    return GDN_OK;
}

}  // namespace

GDN_API gdn_status gdn_prefill_emit_checkpoints_split(const gdn_shape *shape, const void *q,
                                                      const void *k, const void *v,
                                                      const void *alpha, const void *beta,
                                                      const int64_t *h_tok_offset,
                                                      const int64_t *h_first_pos,
                                                      const int64_t *h_ckpt_pos, int32_t M,
                                                      float *ckpt_states, float *state_out, void *o,
                                                      void *workspace, size_t workspace_bytes,
                                                      hipStream_t stream) {
    g_last_error.clear();
    return split_prefill(shape, q, k, v, alpha, beta, h_tok_offset, h_first_pos, h_ckpt_pos, M, ckpt_states,
                         state_out, o, workspace, workspace_bytes, stream);
}

GDN_API gdn_status gdn_prefill_emit_checkpoints_split_noalloc(const gdn_shape *shape, const void *q,
                                                              const void *k, const void *v,
                                                              const void *alpha, const void *beta,
                                                              const int64_t *h_tok_offset,
                                                              const int64_t *h_first_pos,
                                                              const int64_t *h_ckpt_pos, int32_t M,
                                                              float *ckpt_states, float *state_out, void *o,
                                                              hipStream_t stream) {
    g_last_error.clear();
    gdn_status st = check_shape(shape);
    if (st != GDN_OK) return st;
    const size_t need = gdn_prefill_split_workspace_bytes(shape);
    if (need > (size_t)GDN_SPLIT_SCRATCH_BYTES)
        return fail(GDN_ERR_UNSUPPORTED,
                    "the allocation-free split prefill needs %zu bytes of scratch (4 B H d_v d_k floats), more than "
                    "its fixed %zu; use gdn_prefill_emit_checkpoints_split with a workspace",
                    need, (size_t)GDN_SPLIT_SCRATCH_BYTES);
    if (shape->B == 0) return GDN_OK;
    // everything the host can check is checked before the scratch address is taken
    std::vector<Work> probe;
    if ((st = prepare_prefill(shape, h_tok_offset, h_first_pos, h_ckpt_pos, M, ckpt_states, state_out, probe)) !=
        GDN_OK)
        return st;
    if (shape->dk != shape->dv)
        return fail(GDN_ERR_UNSUPPORTED, "the split prefill needs d_k = d_v (got %d, %d)", shape->dk, shape->dv);
    float *ws = nullptr;
    if ((st = scratch_for_current_device(&ws)) != GDN_OK) return st;
    return split_prefill(shape, q, k, v, alpha, beta, h_tok_offset, h_first_pos, h_ckpt_pos, M, ckpt_states,
                         state_out, o, ws, (size_t)GDN_SPLIT_SCRATCH_BYTES, stream);
}
