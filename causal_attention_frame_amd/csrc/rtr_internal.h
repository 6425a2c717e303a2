// Internal interface between the C-ABI host layer (rtr_api.hip) and the HIP
// kernels (attn_fwd.hip, kv_copy.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "rtr_attn.h"

namespace rtr {

// Key frames one streaming call can see: anchored reference + window + chunk.
constexpr int kMaxKeyFrames = RTR_MAX_REF + RTR_MAX_WINDOW + RTR_MAX_CHUNK;
// Frame copies one append can enqueue (K and V of each surviving frame).
constexpr int kMaxCopies = 2 * (RTR_MAX_WINDOW > RTR_MAX_REF ? RTR_MAX_WINDOW : RTR_MAX_REF);

// One attention launch.  Keys are addressed through a segment table: key j lies
// in segment f = j / seg_len, row j - f*seg_len of a [*, H, d] block starting at
// kseg[f] / vseg[f].  The full-sequence form uses one segment holding all keys;
// the streaming form uses one segment per latent frame (reference frames,
// window frames in logical order, then the chunk's frames).
//
// Mask: query row i (0-based within q) may see key j iff
//   j < min(prefix + (floor(i / tokens_per_frame) + 1) * tokens_per_frame, Tk),
// which is the frame mask with `prefix` always-visible cached keys in front.
struct AttnProblem {
    const void *q = nullptr;
    void *o = nullptr;
    float *lse = nullptr;
    const void *kseg[kMaxKeyFrames] = {};
    const void *vseg[kMaxKeyFrames] = {};
    int32_t nseg = 0;
    int64_t seg_len = 0;
    int64_t Tq = 0, Tk = 0;
    int64_t tokens_per_frame = 1;
    int64_t prefix = 0;
    int32_t H = 0, d = 0;
    float scale = 0.f;
    rtr_dtype in_dtype = RTR_BF16, out_dtype = RTR_BF16;
    // Split-K workspace (attention_workspace_bytes() bytes) or null: with it the
    // head_dim-128 bf16 kernel balances the key tiles over the compute units
    // and a second kernel merges the partial results.  ws_slots > 0 caps the
    // partial-result slots a split may use (a workspace of that many slots,
    // kSplitSlotBytes each); 0 means the full attention_workspace_bytes().
    void *ws = nullptr;
    int32_t ws_slots = 0;
};

// Bytes of one partial-result slot of the split launch (256 rows x 128 fp32
// plus two fp32 statistics per row).
constexpr size_t kSplitSlotBytes = (size_t)(256 * 128 + 2 * 256) * sizeof(float);

hipError_t launch_attention(const AttnProblem &p, hipStream_t stream);

// Split-K workspace the attention launch needs on the current device for this
// head dim and input type (0: the launch never splits).
hipError_t attention_workspace_bytes(int32_t d, rtr_dtype in_dtype, size_t *bytes);

// Gradients of the full-sequence form (bf16, head_dim 128).  ws holds
// attention_bwd_workspace_bytes(T, H) bytes: per 32-row tile the log2-domain
// LSE and D of its rows and its transposed Q and dO.
struct BwdProblem {
    const void *q = nullptr, *k = nullptr, *v = nullptr, *o = nullptr, *dout = nullptr;
    const float *lse = nullptr;
    void *dq = nullptr, *dk = nullptr, *dv = nullptr;
    int64_t T = 0, tokens_per_frame = 1;
    int32_t H = 0;
    float scale = 0.f;
    void *ws = nullptr;
    // Streaming step (nseg > 0): q, o, lse, dout and dq hold the chunk's T
    // rows and k, v, dk, dv the chunk's own keys; every key the rows see --
    // `prefix` cached keys, then the chunk's -- also lies in the segment table
    // (as in AttnProblem).  dk_prefix / dv_prefix, when non-null, receive the
    // prefix keys' gradients, [prefix, H, 128].
    const void *kseg[kMaxKeyFrames] = {};
    const void *vseg[kMaxKeyFrames] = {};
    int32_t nseg = 0;
    int64_t seg_len = 0, prefix = 0;
    void *dk_prefix = nullptr, *dv_prefix = nullptr;
    // Cross-attention: the rows have no keys of their own (k, v, dk, dv unused);
    // every key is one of the `prefix` keys of the segment table.
    bool cross = false;
};

// Row groups of a launch of 256-row workgroups (8 waves x 32 rows) over Tq
// query rows of H heads whose key limits follow the frame mask (as in
// AttnProblem): gm 0 = blocks of 256 consecutive rows; gm 2 = 32-row groups
// aligned to frames, frame f paired with frame F-1-f in each workgroup (waves
// 0-3 the early frame's groups, 4-7 the late frame's), the middle frame of an
// odd F in blocks of 8 groups.  gm 2 is chosen only for launches of one round
// on the compute units where it shortens the estimated longest block.  nqb is
// the workgroups per head, wpf the groups per frame, w1 the workgroups per
// frame pair.
struct RowGroups {
    int32_t gm = 0, nqb = 0, wpf = 0, nframes = 0, w1 = 0;
};
hipError_t plan_row_groups(int64_t Tq, int64_t Tk, int64_t kpf, int64_t prefix, int32_t H, RowGroups *out);

hipError_t attention_bwd_workspace_bytes(int64_t T, int32_t H, size_t *bytes);
// Workspace of the cross-attention backward over Tq rows and n text keys:
// the above plus, when the text key blocks are split over the rows, their
// fp32 partial gradients.
hipError_t attention_cross_bwd_workspace_bytes(int64_t Tq, int64_t n, int32_t H, size_t *bytes);
hipError_t launch_attention_bwd(const BwdProblem &p, hipStream_t stream);

// Copies of whole [k, H, d] frames (16-byte multiples, 16-byte aligned).
struct CopyJobs {
    const void *src[kMaxCopies] = {};
    void *dst[kMaxCopies] = {};
    int32_t n = 0;
    int64_t bytes = 0;  // per copy
};

hipError_t launch_frame_copies(const CopyJobs &jobs, hipStream_t stream);

// Temporal rotary re-encoding of `rows` head rows of d elements: pairs
// (2i, 2i+1), i < pairs, rotated by shift * base^(-i / pairs); src and dst are
// 16-byte aligned and either equal (in place) or disjoint.
struct RotateJob {
    const void *src = nullptr;
    void *dst = nullptr;
    int64_t rows = 0;
    int32_t d = 0;
    rtr_dtype dt = RTR_BF16;
    int32_t pairs = 0;
    double base = 10000.0;
    int64_t shift = 0;
};

hipError_t launch_ref_rotate(const RotateJob &j, hipStream_t stream);

// Shader-clock probe: out[0] shader-clock ticks and out[1] 100 MHz ticks over
// about span_ticks of the latter (device buffer of two 64-bit words).
hipError_t launch_clock_probe(unsigned long long *out, int64_t span_ticks, hipStream_t stream);

}  // namespace rtr
