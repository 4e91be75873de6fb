// Launch descriptor passed by value to every replay kernel, and the launcher
// entry points shared by the host code and the kernel translation units.
//
// One launch covers up to kMaxReqPerLaunch work items (a request's span, or
// a segment of it in the split prefill).  Each item contributes H x (d_v / DVB)
// workgroups, one per (item, head, block of DVB value rows).
// The rows of the d_v x d_k state are independent of each other (the key
// operator acts from the right, "Tail-Replay: Escaping the Curse of Linear
// Attention in Prefix Caching for Hybrid LLMs" §2.3), so a (request, head)
// may be split over several workgroups along d_v with no exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kMaxReqPerLaunch = 32;
constexpr int kMaxEmitPerLaunch = 192;

struct LaunchDesc {
    const void *q;
    const void *k;
    const void *v;
    const void *alpha;
    const void *beta;
    void *o;                 // nullable
    const float *init_base;  // start states (resume); offsets below
    float *emit_base;        // emission store [B][M][H][dv][dk] (prefill)
    int32_t H;
    int32_t nreq;            // requests in this launch
    int32_t flags;           // GDN_NORMALIZE_* bits
    int32_t M;               // slots per request in the emission store
    int64_t row0[kMaxReqPerLaunch];      // packed row of the first span token
    int64_t init_off[kMaxReqPerLaunch];  // element offset of (b, slot, head 0) in init_base, -1 = zero
    int32_t len[kMaxReqPerLaunch];       // span length in tokens
    int32_t req[kMaxReqPerLaunch];       // request index b (emission store)
    float *state_dst[kMaxReqPerLaunch];  // final state [H][dv][dk] of the work, NULL: not stored
    int32_t wflags[kMaxReqPerLaunch];    // kWork* bits
    int32_t emit_begin[kMaxReqPerLaunch + 1];
    int32_t emit_after[kMaxEmitPerLaunch];  // span-relative token count, 1..len
    int32_t emit_slot[kMaxEmitPerLaunch];   // slot i in 0..M-1
};

static_assert(sizeof(LaunchDesc) <= 3584, "descriptor must fit the kernel argument segment");

// Flags mirrored from the public header (kept numerically identical).
constexpr int kNormK = 1;
constexpr int kNormQ = 2;
// LaunchDesc::flags bit set by the host (not a public flag): q, k and v are
// one tensor (d_k = d_v), so each row is read once and serves all three.
constexpr int kAliasQKV = 1 << 16;

// Per-work flags (LaunchDesc::wflags).  The sequence-split prefill runs, for a
// middle segment of a span, the zero-start scan (kWorkNoOut) and the product
// of its transitions, which is the same scan with v = 0 started from the
// identity (kWorkZeroV | kWorkNoOut | kWorkIdentity; d_k = d_v).
constexpr int kWorkNoOut = 1;     // no outputs o (nor their stores)
constexpr int kWorkZeroV = 2;     // v taken as zero (v is not read); implies kWorkNoOut
constexpr int kWorkIdentity = 4;  // start state I (init_off is ignored)

enum class Elem : int { F32 = 0, BF16 = 1 };

// Per-token float32 kernel (any supported d_k, d_v; float32 or bf16 storage).
hipError_t launch_recurrent(const LaunchDesc &d, int dk, int dv, Elem e, hipStream_t s);

// Chunked matrix-core kernel; returns hipErrorNotSupported when the shape or
// element type has no chunked variant.
hipError_t launch_chunked(const LaunchDesc &d, int dk, int dv, Elem e, hipStream_t s);

// A group of layers in one launch of the chunked kernel (bf16, d_k = d_v = 128):
// layer 0 reads q, k, v; layer l > 0 reads layer l - 1's outputs as its q = k = v.
constexpr int kMaxGroupLayers = 4;
struct GroupLayer {
    const void *q, *k, *v, *alpha, *beta;
    void *o;
    int64_t state_shift;  // elements added to every state_dst of the descriptor
};
struct GroupPtrs {
    GroupLayer layer[kMaxGroupLayers];
    int32_t L;
};
static_assert(sizeof(LaunchDesc) + sizeof(GroupPtrs) <= 4096, "kernel arguments must fit 4 KiB");
// hipErrorNotSupported unless one launch per layer would run the four-wave
// kernel on every layer (more workgroups than CUs) and o is set.
hipError_t launch_chunked_group(const LaunchDesc &d, const GroupPtrs &g, hipStream_t s);
bool chunked_supported(int dk, int dv, Elem e);

// out = a p + c per pair (a, c, out: [d][d] with d_v = d_k = d; p: [d][d]),
// float32, npairs consecutive pairs; d in {16, 32, 64, 128}.
hipError_t launch_affine_combine(const float *a, const float *p, const float *c, float *out, int64_t npairs, int d,
                                 hipStream_t s);

// Map a hardware workgroup index to a logical one so that consecutive logical
// workgroups land on the same XCD.  Workgroups are handed to the 8 XCDs
// round-robin; logical blocks [x*q + min(x, r), ...) go to XCD x, where
// n = 8q + r.  This is a bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int hw, int n) {
    const int q = n >> 3;
    const int r = n & 7;
    const int x = hw & 7;
    const int slot = hw >> 3;
    return x * q + (x < r ? x : r) + slot;
}

}  // namespace gdn
