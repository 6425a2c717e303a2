// C-ABI host layer of librtr_attn.so: argument checks, the host-side metadata
// of the reference-anchored rolling KV ring, and kernel launches.
//
// The cache semantics follow the RTR-DiT notes ("DiT as Real-Time Rerenderer
// ...", Key Designs 4): a fixed-length window of past latent frames to which
// newly generated frames are appended and from which the oldest are evicted
// once it is full; reference frames held in a separate resident slot in front
// that appending never touches; a condition switch that replaces, keeps or
// clears the reference and keeps only the most recent window frame(s).
//
// Physical layout: window frame slots form a ring over the caller's
// [W, k, H, d] buffers.  Logical position p (0 = oldest) lives in slot
// (head + p) mod W.  Appending into a full ring overwrites slot `head` and
// advances it, so evicting never moves data; trimming on a switch only moves
// `head` and `count`.  Every piece of metadata lives on the host, so no call
// reads device memory or waits for the device.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "rtr_internal.h"

struct rtr_kv_cache {
    void *k_ring, *v_ring, *k_ref, *v_ref;
    int32_t W, N, R_cap;  // window frames, physical ring slots (N >= W), reference capacity
    int64_t kpf;
    int32_t H, d;
    rtr_dtype dt;
    // metadata
    int32_t count, head, ref_frames;
    int64_t ref_gen, next_id;
    int64_t slot_frame_id[RTR_MAX_WINDOW];  // indexed by physical slot
    // The window's count frames occupy slots head, head + 1, ... (mod N).
    // Position-aware reference (rtr_kv_set_ref_rope): the reference K rotated
    // into k_ref_view for the last shift applied, valid while (shift, ref_gen,
    // ref_frames) are unchanged.
    void *k_ref_view = nullptr;
    int32_t rope_pairs = 0;
    double rope_base = 10000.0;
    int64_t pos_offset = 0;
    // (memo of work already enqueued; a const call may update it)
    mutable bool view_valid = false;
    mutable int64_t view_shift = 0, view_gen = -1;
    mutable int32_t view_frames = 0;
};

// One layer's text cross-attention cache (host-side metadata over caller buffers).
struct rtr_text_cache {
    void *k_buf, *v_buf;
    int32_t capacity, H, d;
    rtr_dtype dt;
    int32_t n;        // tokens of the current condition (0: none)
    int64_t gen;      // conditions set so far
};

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    return RTR_OK;
}

constexpr int64_t kMaxTokens = (int64_t)1 << 30;  // token indices stay far from int32 overflow

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
int64_t esize(rtr_dtype dt) { return dt == RTR_BF16 ? 2 : 4; }
bool valid_dtype(int dt) { return dt == RTR_BF16 || dt == RTR_F32; }

bool overlaps(const void *a, int64_t na, const void *b, int64_t nb) {
    if (!a || !b || na <= 0 || nb <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

float resolve_scale(float scale, int d) {
    return (scale > 0.f) ? scale : 1.0f / std::sqrt((float)d);
}

int check_scale(float scale) {
    if (std::isinf(scale)) return fail(RTR_EINVAL, "scale must be finite");
    return RTR_OK;
}

int64_t frame_bytes(const rtr_kv_cache *kv) { return kv->kpf * kv->H * kv->d * esize(kv->dt); }

// One append of a frame to the ring metadata (W window frames over N >= W
// slots); returns the slot written or -1 when W == 0 (nothing is kept).  A
// full window takes the new frame in the slot after its newest and frees its
// oldest: with N == W that is the oldest frame's slot, with N > W a slot the
// window does not use.
int ring_push(int32_t W, int32_t N, int32_t &count, int32_t &head, int64_t &next_id, int64_t *slot_ids) {
    const int64_t id = next_id++;
    if (W == 0) return -1;
    int slot;
    if (count < W) {
        slot = (head + count) % N;
        ++count;
    } else {
        slot = (head + W) % N;
        head = (head + 1) % N;
    }
    slot_ids[slot] = id;
    return slot;
}

// Slots of the next n appends; frames evicted again by the same append get -1.
void plan_append(const rtr_kv_cache *kv, int32_t n, int32_t *slots, int32_t &count, int32_t &head,
                 int64_t &next_id, int64_t *slot_ids) {
    count = kv->count;
    head = kv->head;
    next_id = kv->next_id;
    std::memcpy(slot_ids, kv->slot_frame_id, sizeof(kv->slot_frame_id));
    const int32_t keep_from = n - (n < kv->W ? n : kv->W);  // survivors: f >= n - min(n, W)
    for (int32_t f = 0; f < n; ++f) {
        const int s = ring_push(kv->W, kv->N, count, head, next_id, slot_ids);
        if (slots) slots[f] = (f >= keep_from) ? s : -1;
    }
}

int check_cache(const rtr_kv_cache *kv) {
    if (!kv) return fail(RTR_EINVAL, "cache handle is NULL");
    return RTR_OK;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(RTR_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Checks a split-K workspace against the requirement of the current device and
// the call's other buffers; *use is the pointer to hand to the launch (NULL when
// none is given or the configuration never splits).
int check_workspace(void *ws, size_t ws_bytes, int32_t d, rtr_dtype dt, const void *const *bufs,
                    const int64_t *sizes, int nbufs, void **use, int32_t ws_slots = 0) {
    *use = nullptr;
    if (!ws) return RTR_OK;
    if (!aligned16(ws)) return fail(RTR_EINVAL, "workspace must be 16-byte aligned");
    for (int i = 0; i < nbufs; ++i)
        if (overlaps(ws, (int64_t)ws_bytes, bufs[i], sizes[i]))
            return fail(RTR_EINVAL, "workspace overlaps an input, output or cache buffer");
    size_t need = 0;
    if (const hipError_t e = rtr::attention_workspace_bytes(d, dt, &need)) return hip_fail(e, "workspace size");
    // a slot-capped workspace: the split launch uses at most ws_slots slots
    if (ws_slots > 0 && need > 0) need = std::min(need, (size_t)ws_slots * rtr::kSplitSlotBytes);
    if (ws_bytes < need)
        return fail(RTR_EINVAL, "workspace of %zu bytes, %zu needed on this device", ws_bytes, need);
    *use = need ? ws : nullptr;
    return RTR_OK;
}

// Split-K scratch of rtr_attn_stream_step_noalloc, for callers that cannot
// allocate: a file-scope device array, one copy per GPU the library runs on,
// held until the process ends.  kScratchSlots partial-result slots (34 MB);
// the split planner keeps to that many.  Host code never uses the array's name
// as an address: scratch_ptr() resolves this device's copy once (with the
// device current) and keeps it.
constexpr int32_t kScratchSlots = 256;
constexpr size_t kScratchBytes = (size_t)kScratchSlots * rtr::kSplitSlotBytes;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

int scratch_ptr(void **out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *ptrs[kMaxDevices] = {};
    int dev = 0;
    if (const hipError_t e = hipGetDevice(&dev)) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(RTR_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void *p = nullptr;
        if (const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)))
            return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(RTR_EHIP, "scratch has no device address");
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return RTR_OK;
}

int stream_step(const rtr_kv_cache *kv, const void *q, const void *k, const void *v, void *o, float *lse,
                int32_t chunk_frames, int32_t block_frames, rtr_dtype out_dtype, float scale, void *workspace,
                size_t workspace_bytes, int32_t ws_slots, rtr_stream stream);

}  // namespace

extern "C" {

int rtr_version(void) { return 100; }

const char *rtr_last_error(void) { return g_err.c_str(); }

const char *rtr_status_string(int code) {
    switch (code) {
        case RTR_OK: return "ok";
        case RTR_EINVAL: return "invalid argument";
        case RTR_EUNSUPPORTED: return "unsupported";
        case RTR_EHIP: return "HIP error";
        case RTR_ESTATE: return "invalid cache state";
        default: return "unknown status";
    }
}

int rtr_attn_workspace_size(int32_t d, rtr_dtype in_dtype, size_t *bytes) {
    if (!bytes) return fail(RTR_EINVAL, "bytes is NULL");
    *bytes = 0;
    if (!valid_dtype(in_dtype)) return fail(RTR_EINVAL, "unknown dtype");
    if (d != 64 && d != 128) return fail(RTR_EUNSUPPORTED, "head dim %d not supported (64, 128)", d);
    if (const hipError_t e = rtr::attention_workspace_bytes(d, in_dtype, bytes)) return hip_fail(e, "workspace size");
    return ok();
}

int rtr_attn_block_causal(const void *q, const void *k, const void *v, void *o, float *lse,
                          int64_t T, int32_t H, int32_t d, int64_t tokens_per_frame,
                          rtr_dtype in_dtype, rtr_dtype out_dtype, float scale,
                          void *workspace, size_t workspace_bytes, rtr_stream stream) {
    if (T < 0 || T > kMaxTokens) return fail(RTR_EINVAL, "T=%lld out of range [0, 2^30]", (long long)T);
    if (H < 1) return fail(RTR_EINVAL, "H=%d must be >= 1", H);
    if (tokens_per_frame < 1) return fail(RTR_EINVAL, "tokens_per_frame must be >= 1");
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(RTR_EINVAL, "unknown dtype");
    if (d != 64 && d != 128) return fail(RTR_EUNSUPPORTED, "head dim %d not supported (64, 128)", d);
    if (in_dtype == RTR_F32 && out_dtype != RTR_F32)
        return fail(RTR_EUNSUPPORTED, "float32 input needs float32 output");
    if (int rc = check_scale(scale)) return rc;
    if (T == 0) return ok();
    if (!q || !k || !v || !o) return fail(RTR_EINVAL, "q, k, v and o must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return fail(RTR_EINVAL, "device pointers must be 16-byte aligned");
    const int64_t in_bytes = T * H * d * esize(in_dtype);
    const int64_t out_bytes = T * H * d * esize(out_dtype);
    const int64_t lse_bytes = T * H * 4;
    for (const void *x : {q, k, v}) {
        if (overlaps(o, out_bytes, x, in_bytes)) return fail(RTR_EINVAL, "o overlaps an input");
        if (overlaps(lse, lse_bytes, x, in_bytes)) return fail(RTR_EINVAL, "lse overlaps an input");
    }
    if (overlaps(lse, lse_bytes, o, out_bytes)) return fail(RTR_EINVAL, "lse overlaps o");
    void *ws = nullptr;
    {
        const void *bufs[5] = {q, k, v, o, lse};
        const int64_t sizes[5] = {in_bytes, in_bytes, in_bytes, out_bytes, lse ? lse_bytes : 0};
        if (int rc = check_workspace(workspace, workspace_bytes, d, in_dtype, bufs, sizes, 5, &ws)) return rc;
    }

    rtr::AttnProblem p;
    p.ws = ws;
    p.q = q;
    p.o = o;
    p.lse = lse;
    p.kseg[0] = k;
    p.vseg[0] = v;
    p.nseg = 1;
    p.seg_len = T;
    p.Tq = T;
    p.Tk = T;
    p.tokens_per_frame = tokens_per_frame < T ? tokens_per_frame : T;
    p.prefix = 0;
    p.H = H;
    p.d = d;
    p.scale = resolve_scale(scale, d);
    p.in_dtype = in_dtype;
    p.out_dtype = out_dtype;
    const hipError_t e = rtr::launch_attention(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    return ok();
}

int rtr_attn_bwd_workspace_size(int64_t T, int32_t H, int32_t d, size_t *bytes) {
    if (!bytes) return fail(RTR_EINVAL, "bytes is NULL");
    *bytes = 0;
    if (T < 0 || T > kMaxTokens) return fail(RTR_EINVAL, "T=%lld out of range [0, 2^30]", (long long)T);
    if (H < 1) return fail(RTR_EINVAL, "H=%d must be >= 1", H);
    if (d != 128) return fail(RTR_EUNSUPPORTED, "backward head dim %d not supported (128)", d);
    if (const hipError_t e = rtr::attention_bwd_workspace_bytes(T, H, bytes)) return hip_fail(e, "workspace size");
    return ok();
}

int rtr_attn_block_causal_bwd(const void *q, const void *k, const void *v, const void *o,
                              const float *lse, const void *d_o, void *dq, void *dk, void *dv,
                              int64_t T, int32_t H, int32_t d, int64_t tokens_per_frame,
                              rtr_dtype dtype, float scale, void *workspace,
                              size_t workspace_bytes, rtr_stream stream) {
    if (T < 0 || T > kMaxTokens) return fail(RTR_EINVAL, "T=%lld out of range [0, 2^30]", (long long)T);
    if (H < 1) return fail(RTR_EINVAL, "H=%d must be >= 1", H);
    if (tokens_per_frame < 1) return fail(RTR_EINVAL, "tokens_per_frame must be >= 1");
    if (!valid_dtype(dtype)) return fail(RTR_EINVAL, "unknown dtype");
    if (dtype != RTR_BF16) return fail(RTR_EUNSUPPORTED, "backward supports bf16 only");
    if (d != 128) return fail(RTR_EUNSUPPORTED, "backward head dim %d not supported (128)", d);
    if (T * H * d >= ((int64_t)1 << 31)) return fail(RTR_EUNSUPPORTED, "T * H * d must be below 2^31");
    if (int rc = check_scale(scale)) return rc;
    if (T == 0) return ok();
    const void *in[6] = {q, k, v, o, lse, d_o};
    void *out[3] = {dq, dk, dv};
    for (const void *x : in)
        if (!x) return fail(RTR_EINVAL, "q, k, v, o, lse and d_o must be non-NULL");
    for (const void *x : out)
        if (!x) return fail(RTR_EINVAL, "dq, dk and dv must be non-NULL");
    for (const void *x : {q, k, v, o, d_o, (const void *)dq, (const void *)dk, (const void *)dv})
        if (!aligned16(x)) return fail(RTR_EINVAL, "tensor pointers must be 16-byte aligned");
    if (((uintptr_t)lse & 3u) != 0) return fail(RTR_EINVAL, "lse must be 4-byte aligned");
    const int64_t tb = T * H * d * 2, lb = T * H * 4;
    const int64_t in_sz[6] = {tb, tb, tb, tb, lb, tb};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(out[i], tb, in[j], in_sz[j])) return fail(RTR_EINVAL, "an output overlaps an input");
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(out[i], tb, out[j], tb)) return fail(RTR_EINVAL, "outputs overlap");
    }
    size_t need = 0;
    if (const hipError_t e = rtr::attention_bwd_workspace_bytes(T, H, &need)) return hip_fail(e, "workspace size");
    if (!workspace) return fail(RTR_EINVAL, "workspace is NULL (%zu bytes needed)", need);
    if (((uintptr_t)workspace & 255u) != 0) return fail(RTR_EINVAL, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
        return fail(RTR_EINVAL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    for (int j = 0; j < 6; ++j)
        if (overlaps(workspace, (int64_t)need, in[j], in_sz[j])) return fail(RTR_EINVAL, "workspace overlaps an input");
    for (int i = 0; i < 3; ++i)
        if (overlaps(workspace, (int64_t)need, out[i], tb)) return fail(RTR_EINVAL, "workspace overlaps an output");

    rtr::BwdProblem p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = d_o;
    p.lse = lse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.T = T;
    p.tokens_per_frame = tokens_per_frame;
    p.H = H;
    p.scale = resolve_scale(scale, d);
    p.ws = workspace;
    const hipError_t e = rtr::launch_attention_bwd(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return ok();
}

int rtr_kv_create(rtr_kv_cache **out, void *k_ring, void *v_ring, void *k_ref, void *v_ref,
                  int32_t window_frames, int32_t ref_capacity_frames, int64_t tokens_per_frame,
                  int32_t H, int32_t d, rtr_dtype dtype) {
    return rtr_kv_create_slots(out, k_ring, v_ring, k_ref, v_ref, window_frames, window_frames,
                               ref_capacity_frames, tokens_per_frame, H, d, dtype);
}

int rtr_kv_create_slots(rtr_kv_cache **out, void *k_ring, void *v_ring, void *k_ref, void *v_ref,
                        int32_t window_frames, int32_t ring_slots, int32_t ref_capacity_frames,
                        int64_t tokens_per_frame, int32_t H, int32_t d, rtr_dtype dtype) {
    if (!out) return fail(RTR_EINVAL, "out is NULL");
    if (window_frames < 0 || window_frames > RTR_MAX_WINDOW)
        return fail(RTR_EUNSUPPORTED, "window_frames=%d outside [0, %d]", window_frames, RTR_MAX_WINDOW);
    if (ring_slots < window_frames || ring_slots > RTR_MAX_WINDOW)
        return fail(RTR_EUNSUPPORTED, "ring_slots=%d outside [window_frames=%d, %d]", ring_slots, window_frames,
                    RTR_MAX_WINDOW);
    if (ref_capacity_frames < 0 || ref_capacity_frames > RTR_MAX_REF)
        return fail(RTR_EUNSUPPORTED, "ref_capacity_frames=%d outside [0, %d]", ref_capacity_frames,
                    RTR_MAX_REF);
    if (tokens_per_frame < 1) return fail(RTR_EINVAL, "tokens_per_frame must be >= 1");
    if (H < 1) return fail(RTR_EINVAL, "H must be >= 1");
    if (!valid_dtype(dtype)) return fail(RTR_EINVAL, "unknown dtype");
    if (d != 64 && d != 128) return fail(RTR_EUNSUPPORTED, "head dim %d not supported (64, 128)", d);
    const int64_t total_frames = (int64_t)RTR_MAX_REF + RTR_MAX_WINDOW + RTR_MAX_CHUNK;
    if (tokens_per_frame * total_frames > kMaxTokens)
        return fail(RTR_EUNSUPPORTED, "tokens_per_frame too large");
    if (window_frames > 0 && (!k_ring || !v_ring))
        return fail(RTR_EINVAL, "ring buffers must be non-NULL when window_frames > 0");
    if (ref_capacity_frames > 0 && (!k_ref || !v_ref))
        return fail(RTR_EINVAL, "reference buffers must be non-NULL when ref capacity > 0");
    if (!aligned16(k_ring) || !aligned16(v_ring) || !aligned16(k_ref) || !aligned16(v_ref))
        return fail(RTR_EINVAL, "cache buffers must be 16-byte aligned");
    const int64_t fb = tokens_per_frame * H * d * esize(dtype);
    const int64_t ring_b = fb * ring_slots, ref_b = fb * ref_capacity_frames;
    const void *bufs[4] = {k_ring, v_ring, k_ref, v_ref};
    const int64_t sizes[4] = {ring_b, ring_b, ref_b, ref_b};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(bufs[i], sizes[i], bufs[j], sizes[j]))
                return fail(RTR_EINVAL, "cache buffers overlap");

    rtr_kv_cache *kv = new (std::nothrow) rtr_kv_cache();
    if (!kv) return fail(RTR_EINVAL, "out of host memory");
    kv->k_ring = k_ring;
    kv->v_ring = v_ring;
    kv->k_ref = k_ref;
    kv->v_ref = v_ref;
    kv->W = window_frames;
    kv->N = ring_slots;
    kv->R_cap = ref_capacity_frames;
    kv->kpf = tokens_per_frame;
    kv->H = H;
    kv->d = d;
    kv->dt = dtype;
    kv->count = 0;
    kv->head = 0;
    kv->ref_frames = 0;
    kv->ref_gen = 0;
    kv->next_id = 0;
    for (auto &x : kv->slot_frame_id) x = -1;
    *out = kv;
    return ok();
}

int rtr_kv_destroy(rtr_kv_cache *kv) {
    delete kv;
    return ok();
}

int rtr_kv_next_slots(const rtr_kv_cache *kv, int32_t n_frames, int32_t *slots) {
    if (int rc = check_cache(kv)) return rc;
    if (n_frames < 0) return fail(RTR_EINVAL, "n_frames must be >= 0");
    if (n_frames > 0 && !slots) return fail(RTR_EINVAL, "slots is NULL");
    int32_t count, head;
    int64_t next_id, ids[RTR_MAX_WINDOW];
    plan_append(kv, n_frames, slots, count, head, next_id, ids);
    return ok();
}

int rtr_kv_commit_inplace(rtr_kv_cache *kv, int32_t n_frames) {
    if (int rc = check_cache(kv)) return rc;
    if (n_frames < 0) return fail(RTR_EINVAL, "n_frames must be >= 0");
    int32_t count, head;
    int64_t next_id, ids[RTR_MAX_WINDOW];
    plan_append(kv, n_frames, nullptr, count, head, next_id, ids);
    kv->count = count;
    kv->head = head;
    kv->next_id = next_id;
    std::memcpy(kv->slot_frame_id, ids, sizeof ids);
    return ok();
}

int rtr_kv_append_evict(rtr_kv_cache *kv, const void *k_new, const void *v_new, int32_t n_frames,
                        rtr_stream stream) {
    if (int rc = check_cache(kv)) return rc;
    if (n_frames < 0) return fail(RTR_EINVAL, "n_frames must be >= 0");
    if (n_frames == 0) return ok();
    if (!k_new || !v_new) return fail(RTR_EINVAL, "k_new and v_new must be non-NULL");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(RTR_EINVAL, "k_new/v_new must be 16-byte aligned");
    const int64_t fb = frame_bytes(kv);
    const int64_t nb = fb * n_frames;
    const int64_t ring_b = fb * kv->N;
    for (const void *src : {k_new, v_new})
        for (const void *dst : {kv->k_ring, kv->v_ring})
            if (overlaps(src, nb, dst, ring_b)) return fail(RTR_EINVAL, "new frames overlap the ring buffers");

    // Frames f < n - min(n, W) are evicted again by this same append: they get
    // ids but are never copied.
    const int32_t survivors = n_frames < kv->W ? n_frames : kv->W;
    const int32_t first = n_frames - survivors;
    int32_t slots[RTR_MAX_WINDOW];
    int32_t count = kv->count, head = kv->head;
    int64_t next_id = kv->next_id, ids[RTR_MAX_WINDOW];
    std::memcpy(ids, kv->slot_frame_id, sizeof ids);
    for (int32_t f = 0; f < n_frames; ++f) {
        const int s = ring_push(kv->W, kv->N, count, head, next_id, ids);
        if (f >= first) slots[f - first] = s;
    }
    rtr::CopyJobs jobs;
    for (int32_t f = 0; f < survivors; ++f) {
        const int64_t src_off = (int64_t)(first + f) * fb;
        const int64_t dst_off = (int64_t)slots[f] * fb;
        jobs.src[jobs.n] = (const char *)k_new + src_off;
        jobs.dst[jobs.n++] = (char *)kv->k_ring + dst_off;
        jobs.src[jobs.n] = (const char *)v_new + src_off;
        jobs.dst[jobs.n++] = (char *)kv->v_ring + dst_off;
    }
    jobs.bytes = fb;
    if (jobs.n > 0) {
        const hipError_t e = rtr::launch_frame_copies(jobs, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "ring copy launch");
    }
    kv->count = count;
    kv->head = head;
    kv->next_id = next_id;
    std::memcpy(kv->slot_frame_id, ids, sizeof ids);
    return ok();
}

int rtr_kv_reset_ref(rtr_kv_cache *kv, rtr_ref_mode mode, const void *k_ref, const void *v_ref,
                     int32_t ref_frames, int32_t keep_recent, rtr_stream stream) {
    if (int rc = check_cache(kv)) return rc;
    if (mode != RTR_REF_KEEP && mode != RTR_REF_REPLACE && mode != RTR_REF_CLEAR)
        return fail(RTR_EINVAL, "unknown reference mode %d", (int)mode);
    if (keep_recent < -1) return fail(RTR_EINVAL, "keep_recent must be >= -1");
    const int64_t fb = frame_bytes(kv);
    bool copy = false;
    if (mode == RTR_REF_REPLACE) {
        if (kv->R_cap < 1) return fail(RTR_ESTATE, "cache was created without reference capacity");
        if (ref_frames < 1 || ref_frames > kv->R_cap)
            return fail(RTR_EINVAL, "ref_frames=%d outside [1, %d]", ref_frames, kv->R_cap);
        if ((k_ref == nullptr) != (v_ref == nullptr))
            return fail(RTR_EINVAL, "k_ref and v_ref must both be NULL or both non-NULL");
        if (k_ref) {
            if (!aligned16(k_ref) || !aligned16(v_ref)) return fail(RTR_EINVAL, "reference pointers must be 16-byte aligned");
            const int64_t nb = fb * ref_frames;
            const bool same = (k_ref == kv->k_ref && v_ref == kv->v_ref);
            if (!same) {
                for (const void *src : {k_ref, v_ref}) {
                    for (const void *dst : {kv->k_ref, kv->v_ref})
                        if (overlaps(src, nb, dst, fb * kv->R_cap))
                            return fail(RTR_EINVAL, "new reference overlaps the reference slot");
                    for (const void *dst : {kv->k_ring, kv->v_ring})
                        if (overlaps(src, nb, dst, fb * kv->N))
                            return fail(RTR_EINVAL, "new reference overlaps the ring buffers");
                }
                copy = true;
            }
        }
    }
    if (copy) {
        rtr::CopyJobs jobs;
        jobs.src[0] = k_ref;
        jobs.dst[0] = kv->k_ref;
        jobs.src[1] = v_ref;
        jobs.dst[1] = kv->v_ref;
        jobs.n = 2;
        jobs.bytes = fb * ref_frames;
        const hipError_t e = rtr::launch_frame_copies(jobs, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "reference copy launch");
    }
    if (mode == RTR_REF_REPLACE) {
        kv->ref_frames = ref_frames;
        ++kv->ref_gen;
    } else if (mode == RTR_REF_CLEAR) {
        kv->ref_frames = 0;
    }
    if (keep_recent >= 0 && keep_recent < kv->count) {
        kv->head = (kv->head + kv->count - keep_recent) % kv->N;
        kv->count = keep_recent;
    }
    return ok();
}

namespace {

// Position-aware reference (rtr_kv_set_ref_rope): the rotation applied to the
// reference K for the current cache state -- the reference sits right in front
// of the oldest frame a step sees.
int64_t ref_shift(const rtr_kv_cache *kv) {
    const int64_t oldest = (kv->count > 0 ? kv->slot_frame_id[kv->head] : kv->next_id) + kv->pos_offset;
    return oldest - kv->ref_frames;
}

// Reference keys a step attends to: the stored ones, or their rotated view,
// re-rotated only when the shift or the reference has changed since the last
// rotation enqueued.
int ref_keys(const rtr_kv_cache *kv, hipStream_t stream, const void **kref) {
    *kref = kv->k_ref;
    if (!(kv->k_ref_view && kv->ref_frames > 0)) return RTR_OK;
    const int64_t shift = ref_shift(kv);
    if (!(kv->view_valid && kv->view_shift == shift && kv->view_gen == kv->ref_gen &&
          kv->view_frames == kv->ref_frames)) {
        rtr::RotateJob j;
        j.src = kv->k_ref;
        j.dst = kv->k_ref_view;
        j.rows = (int64_t)kv->ref_frames * kv->kpf * kv->H;
        j.d = kv->d;
        j.dt = kv->dt;
        j.pairs = kv->rope_pairs;
        j.base = kv->rope_base;
        j.shift = shift;
        if (const hipError_t e = rtr::launch_ref_rotate(j, stream)) return hip_fail(e, "reference rotation launch");
        kv->view_valid = true;
        kv->view_shift = shift;
        kv->view_gen = kv->ref_gen;
        kv->view_frames = kv->ref_frames;
    }
    *kref = kv->k_ref_view;
    return RTR_OK;
}

// Key segment table of a step, one latent frame per segment: the reference
// frames, the window frames oldest first, then the chunk's frames.
int key_segments(const rtr_kv_cache *kv, const void *kref, const void *k, const void *v, int32_t chunk_frames,
                 const void **kseg, const void **vseg) {
    const int64_t fb = frame_bytes(kv);
    int nseg = 0;
    for (int r = 0; r < kv->ref_frames; ++r) {
        kseg[nseg] = (const char *)kref + r * fb;
        vseg[nseg++] = (const char *)kv->v_ref + r * fb;
    }
    for (int i = 0; i < kv->count; ++i) {
        const int slot = (kv->head + i) % kv->N;
        kseg[nseg] = (const char *)kv->k_ring + slot * fb;
        vseg[nseg++] = (const char *)kv->v_ring + slot * fb;
    }
    for (int c = 0; c < chunk_frames; ++c) {
        kseg[nseg] = (const char *)k + c * fb;
        vseg[nseg++] = (const char *)v + c * fb;
    }
    return nseg;
}

// Whether [p, p + nb) overlaps memory that a step reads from the cache: a
// window slot in use (the ring's other slots may hold a chunk that a producer
// writes there before committing it in place), or the reference slot and its
// rotated view.  A chunk placed there would be read twice, once as cached keys.
bool aliases_cache(const rtr_kv_cache *kv, const void *p, int64_t nb) {
    const int64_t fb = frame_bytes(kv);
    for (int i = 0; i < kv->count; ++i) {
        const int64_t off = (int64_t)((kv->head + i) % kv->N) * fb;
        if (overlaps(p, nb, (const char *)kv->k_ring + off, fb) || overlaps(p, nb, (const char *)kv->v_ring + off, fb))
            return true;
    }
    return overlaps(p, nb, kv->k_ref, fb * kv->R_cap) || overlaps(p, nb, kv->v_ref, fb * kv->R_cap) ||
           (kv->k_ref_view && overlaps(p, nb, kv->k_ref_view, fb * kv->R_cap));
}

}  // namespace

int rtr_attn_stream_step(const rtr_kv_cache *kv, const void *q, const void *k, const void *v,
                         void *o, float *lse, int32_t chunk_frames, rtr_dtype out_dtype,
                         float scale, void *workspace, size_t workspace_bytes,
                         rtr_stream stream) {
    return rtr_attn_stream_step_blocked(kv, q, k, v, o, lse, chunk_frames, 1, out_dtype, scale, workspace,
                                        workspace_bytes, stream);
}

int rtr_attn_stream_step_blocked(const rtr_kv_cache *kv, const void *q, const void *k, const void *v,
                                 void *o, float *lse, int32_t chunk_frames, int32_t block_frames,
                                 rtr_dtype out_dtype, float scale, void *workspace,
                                 size_t workspace_bytes, rtr_stream stream) {
    return stream_step(kv, q, k, v, o, lse, chunk_frames, block_frames, out_dtype, scale, workspace,
                       workspace_bytes, 0, stream);
}

int rtr_attn_stream_step_noalloc(const rtr_kv_cache *kv, const void *q, const void *k, const void *v,
                                 void *o, float *lse, int32_t chunk_frames, int32_t block_frames,
                                 rtr_dtype out_dtype, float scale, rtr_stream stream) {
    void *ws = nullptr;
    if (int rc = scratch_ptr(&ws)) return rc;
    return stream_step(kv, q, k, v, o, lse, chunk_frames, block_frames, out_dtype, scale, ws,
                       kScratchBytes, kScratchSlots, stream);
}

}  // extern "C"

namespace {

int stream_step(const rtr_kv_cache *kv, const void *q, const void *k, const void *v, void *o, float *lse,
                int32_t chunk_frames, int32_t block_frames, rtr_dtype out_dtype, float scale, void *workspace,
                size_t workspace_bytes, int32_t ws_slots, rtr_stream stream) {
    if (int rc = check_cache(kv)) return rc;
    if (chunk_frames < 1 || chunk_frames > RTR_MAX_CHUNK)
        return fail(RTR_EUNSUPPORTED, "chunk_frames=%d outside [1, %d]", chunk_frames, RTR_MAX_CHUNK);
    if (block_frames < 1) return fail(RTR_EINVAL, "block_frames=%d must be >= 1", block_frames);
    const int32_t mask_frames = block_frames < chunk_frames ? block_frames : chunk_frames;
    if (!valid_dtype(out_dtype)) return fail(RTR_EINVAL, "unknown dtype");
    if (kv->dt == RTR_F32 && out_dtype != RTR_F32)
        return fail(RTR_EUNSUPPORTED, "float32 cache needs float32 output");
    if (int rc = check_scale(scale)) return rc;
    if (!q || !k || !v || !o) return fail(RTR_EINVAL, "q, k, v and o must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return fail(RTR_EINVAL, "device pointers must be 16-byte aligned");
    const int64_t fb = frame_bytes(kv);
    const int64_t Tq = (int64_t)chunk_frames * kv->kpf;
    const int64_t in_b = fb * chunk_frames;
    for (const void *x : {q, k, v})
        if (aliases_cache(kv, x, in_b))
            return fail(RTR_EINVAL, "q, k or v overlaps a window slot or the reference that the step reads");
    const int64_t out_b = Tq * kv->H * kv->d * esize(out_dtype);
    const int64_t lse_b = Tq * kv->H * 4;
    const void *ins[8] = {q, k, v, kv->k_ring, kv->v_ring, kv->k_ref, kv->v_ref, kv->k_ref_view};
    const int64_t in_sz[8] = {in_b, in_b, in_b, fb * kv->N, fb * kv->N, fb * kv->R_cap, fb * kv->R_cap,
                              kv->k_ref_view ? fb * kv->R_cap : 0};
    for (int i = 0; i < 8; ++i) {
        if (overlaps(o, out_b, ins[i], in_sz[i])) return fail(RTR_EINVAL, "o overlaps an input or the cache");
        if (overlaps(lse, lse_b, ins[i], in_sz[i])) return fail(RTR_EINVAL, "lse overlaps an input or the cache");
    }
    if (overlaps(lse, lse_b, o, out_b)) return fail(RTR_EINVAL, "lse overlaps o");
    void *ws = nullptr;
    {
        const void *bufs[9] = {q, k, v, kv->k_ring, kv->v_ring, kv->k_ref, kv->v_ref, o, lse};
        const int64_t sizes[9] = {in_b, in_b, in_b, fb * kv->N, fb * kv->N, fb * kv->R_cap, fb * kv->R_cap,
                                  out_b, lse ? lse_b : 0};
        if (int rc = check_workspace(workspace, workspace_bytes, kv->d, kv->dt, bufs, sizes, 9, &ws, ws_slots))
            return rc;
    }

    const void *kref = nullptr;
    if (int rc = ref_keys(kv, (hipStream_t)stream, &kref)) return rc;

    rtr::AttnProblem p;
    p.ws = ws;
    p.ws_slots = ws_slots;
    const int nseg = key_segments(kv, kref, k, v, chunk_frames, p.kseg, p.vseg);
    p.q = q;
    p.o = o;
    p.lse = lse;
    p.nseg = nseg;
    p.seg_len = kv->kpf;
    p.Tq = Tq;
    p.prefix = (int64_t)(kv->ref_frames + kv->count) * kv->kpf;
    p.Tk = p.prefix + Tq;
    p.tokens_per_frame = (int64_t)mask_frames * kv->kpf;  // mask unit; segments stay one frame
    p.H = kv->H;
    p.d = kv->d;
    p.scale = resolve_scale(scale, kv->d);
    p.in_dtype = kv->dt;
    p.out_dtype = out_dtype;
    const hipError_t e = rtr::launch_attention(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    return ok();
}

}  // namespace

extern "C" {

int rtr_attn_stream_step_bwd(const rtr_kv_cache *kv, const void *q, const void *k, const void *v,
                             const void *o, const float *lse, const void *d_o, int32_t chunk_frames,
                             int32_t block_frames, void *dq, void *dk, void *dv, void *dk_cache,
                             void *dv_cache, float scale, void *workspace, size_t workspace_bytes,
                             rtr_stream stream) {
    if (int rc = check_cache(kv)) return rc;
    if (kv->dt != RTR_BF16) return fail(RTR_EUNSUPPORTED, "backward supports bf16 only");
    if (kv->d != 128) return fail(RTR_EUNSUPPORTED, "backward head dim %d not supported (128)", kv->d);
    if (chunk_frames < 1 || chunk_frames > RTR_MAX_CHUNK)
        return fail(RTR_EUNSUPPORTED, "chunk_frames=%d outside [1, %d]", chunk_frames, RTR_MAX_CHUNK);
    if (block_frames < 1) return fail(RTR_EINVAL, "block_frames=%d must be >= 1", block_frames);
    if (int rc = check_scale(scale)) return rc;
    const int32_t mask_frames = block_frames < chunk_frames ? block_frames : chunk_frames;
    const int64_t Tq = (int64_t)chunk_frames * kv->kpf;
    const int64_t P = (int64_t)(kv->ref_frames + kv->count) * kv->kpf;
    if (Tq * kv->H * kv->d >= ((int64_t)1 << 31)) return fail(RTR_EUNSUPPORTED, "chunk tokens * H * d must be below 2^31");
    if ((dk_cache == nullptr) != (dv_cache == nullptr))
        return fail(RTR_EINVAL, "dk_cache and dv_cache must both be NULL or both non-NULL");
    const void *in[6] = {q, k, v, o, lse, d_o};
    for (const void *x : in)
        if (!x) return fail(RTR_EINVAL, "q, k, v, o, lse and d_o must be non-NULL");
    void *out[5] = {dq, dk, dv, dk_cache, dv_cache};
    for (int i = 0; i < 3; ++i)
        if (!out[i]) return fail(RTR_EINVAL, "dq, dk and dv must be non-NULL");
    for (const void *x : {q, k, v, o, d_o, (const void *)dq, (const void *)dk, (const void *)dv,
                          (const void *)dk_cache, (const void *)dv_cache})
        if (!aligned16(x)) return fail(RTR_EINVAL, "tensor pointers must be 16-byte aligned");
    if (((uintptr_t)lse & 3u) != 0) return fail(RTR_EINVAL, "lse must be 4-byte aligned");
    const int64_t fb = frame_bytes(kv);
    const int64_t tb = fb * chunk_frames, lb = Tq * kv->H * 4, pb = P * kv->H * kv->d * 2;
    for (const void *x : {q, k, v, o, d_o})
        if (aliases_cache(kv, x, tb))
            return fail(RTR_EINVAL, "q, k, v, o or d_o overlaps a window slot or the reference that the step reads");
    const int64_t out_sz[5] = {tb, tb, tb, dk_cache ? pb : 0, dv_cache ? pb : 0};
    const void *src[10] = {q, k, v, o, lse, d_o, kv->k_ring, kv->v_ring, kv->k_ref, kv->v_ref};
    const int64_t src_sz[10] = {tb, tb, tb, tb, lb, tb, fb * kv->N, fb * kv->N, fb * kv->R_cap, fb * kv->R_cap};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 10; ++j)
            if (overlaps(out[i], out_sz[i], src[j], src_sz[j])) return fail(RTR_EINVAL, "an output overlaps an input or the cache");
        if (kv->k_ref_view && overlaps(out[i], out_sz[i], kv->k_ref_view, fb * kv->R_cap))
            return fail(RTR_EINVAL, "an output overlaps the rotated reference");
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(out[i], out_sz[i], out[j], out_sz[j])) return fail(RTR_EINVAL, "outputs overlap");
    }
    size_t need = 0;
    if (const hipError_t e = rtr::attention_bwd_workspace_bytes(Tq, kv->H, &need)) return hip_fail(e, "workspace size");
    if (!workspace) return fail(RTR_EINVAL, "workspace is NULL (%zu bytes needed)", need);
    if (((uintptr_t)workspace & 255u) != 0) return fail(RTR_EINVAL, "workspace must be 256-byte aligned");
    if (workspace_bytes < need) return fail(RTR_EINVAL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    for (int j = 0; j < 10; ++j)
        if (overlaps(workspace, (int64_t)need, src[j], src_sz[j])) return fail(RTR_EINVAL, "workspace overlaps an input or the cache");
    for (int i = 0; i < 5; ++i)
        if (overlaps(workspace, (int64_t)need, out[i], out_sz[i])) return fail(RTR_EINVAL, "workspace overlaps an output");
    if (kv->k_ref_view && overlaps(workspace, (int64_t)need, kv->k_ref_view, fb * kv->R_cap))
        return fail(RTR_EINVAL, "workspace overlaps the rotated reference");

    const void *kref = nullptr;
    if (int rc = ref_keys(kv, (hipStream_t)stream, &kref)) return rc;
    rtr::BwdProblem p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = d_o;
    p.lse = lse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.T = Tq;
    p.tokens_per_frame = (int64_t)mask_frames * kv->kpf;
    p.H = kv->H;
    p.scale = resolve_scale(scale, kv->d);
    p.ws = workspace;
    p.nseg = key_segments(kv, kref, k, v, chunk_frames, p.kseg, p.vseg);
    p.seg_len = kv->kpf;
    p.prefix = P;
    if (dk_cache && P > 0) {
        p.dk_prefix = dk_cache;
        p.dv_prefix = dv_cache;
    }
    if (const hipError_t e = rtr::launch_attention_bwd(p, (hipStream_t)stream)) return hip_fail(e, "backward launch");
    // A rotated reference: its keys' gradient so far is with respect to the
    // rotated view; the rotation is orthogonal, so rotating back by the same
    // angle gives the gradient with respect to the stored keys.
    if (dk_cache && P > 0 && kref != kv->k_ref) {
        rtr::RotateJob j;
        j.src = dk_cache;
        j.dst = dk_cache;
        j.rows = (int64_t)kv->ref_frames * kv->kpf * kv->H;
        j.d = kv->d;
        j.dt = kv->dt;
        j.pairs = kv->rope_pairs;
        j.base = kv->rope_base;
        j.shift = -kv->view_shift;
        if (const hipError_t e = rtr::launch_ref_rotate(j, (hipStream_t)stream)) return hip_fail(e, "gradient rotation launch");
    }
    return ok();
}

int rtr_text_cache_create(rtr_text_cache **out, void *k_buf, void *v_buf, int32_t capacity_tokens,
                          int32_t H, int32_t d, rtr_dtype dtype) {
    if (!out) return fail(RTR_EINVAL, "out is NULL");
    if (capacity_tokens < 1 || capacity_tokens > kMaxTokens)
        return fail(RTR_EINVAL, "capacity_tokens=%d must be >= 1", capacity_tokens);
    if (H < 1) return fail(RTR_EINVAL, "H must be >= 1");
    if (!valid_dtype(dtype)) return fail(RTR_EINVAL, "unknown dtype");
    if (d != 64 && d != 128) return fail(RTR_EUNSUPPORTED, "head dim %d not supported (64, 128)", d);
    if (!k_buf || !v_buf) return fail(RTR_EINVAL, "cache buffers must be non-NULL");
    if (!aligned16(k_buf) || !aligned16(v_buf)) return fail(RTR_EINVAL, "cache buffers must be 16-byte aligned");
    const int64_t nb = (int64_t)capacity_tokens * H * d * esize(dtype);
    if (overlaps(k_buf, nb, v_buf, nb)) return fail(RTR_EINVAL, "cache buffers overlap");
    rtr_text_cache *tc = new (std::nothrow) rtr_text_cache();
    if (!tc) return fail(RTR_EINVAL, "out of host memory");
    tc->k_buf = k_buf;
    tc->v_buf = v_buf;
    tc->capacity = capacity_tokens;
    tc->H = H;
    tc->d = d;
    tc->dt = dtype;
    tc->n = 0;
    tc->gen = 0;
    *out = tc;
    return ok();
}

int rtr_text_cache_destroy(rtr_text_cache *tc) {
    delete tc;
    return ok();
}

int rtr_text_cache_reset(rtr_text_cache *tc, const void *k_text, const void *v_text, int32_t n_tokens,
                         rtr_stream stream) {
    if (!tc) return fail(RTR_EINVAL, "cache handle is NULL");
    if (n_tokens < 0 || n_tokens > tc->capacity)
        return fail(RTR_EINVAL, "n_tokens=%d outside [0, %d]", n_tokens, tc->capacity);
    if ((k_text == nullptr) != (v_text == nullptr))
        return fail(RTR_EINVAL, "k_text and v_text must both be NULL or both non-NULL");
    if (n_tokens == 0) {
        tc->n = 0;
        return ok();
    }
    const int64_t tok_b = (int64_t)tc->H * tc->d * esize(tc->dt);
    if (k_text && !(k_text == tc->k_buf && v_text == tc->v_buf)) {
        if (!aligned16(k_text) || !aligned16(v_text)) return fail(RTR_EINVAL, "text pointers must be 16-byte aligned");
        const int64_t nb = tok_b * n_tokens, cap_b = tok_b * tc->capacity;
        for (const void *src : {k_text, v_text})
            for (const void *dst : {tc->k_buf, tc->v_buf})
                if (overlaps(src, nb, dst, cap_b)) return fail(RTR_EINVAL, "new text K/V overlaps the cache buffers");
        rtr::CopyJobs jobs;
        jobs.src[0] = k_text;
        jobs.dst[0] = tc->k_buf;
        jobs.src[1] = v_text;
        jobs.dst[1] = tc->v_buf;
        jobs.n = 2;
        jobs.bytes = nb;
        const hipError_t e = rtr::launch_frame_copies(jobs, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "text copy launch");
    }
    tc->n = n_tokens;
    ++tc->gen;
    return ok();
}

int rtr_text_cache_state(const rtr_text_cache *tc, int32_t *n_tokens, int64_t *generation) {
    if (!tc) return fail(RTR_EINVAL, "cache handle is NULL");
    if (n_tokens) *n_tokens = tc->n;
    if (generation) *generation = tc->gen;
    return ok();
}

int rtr_attn_cross_bwd_workspace_size(int64_t Tq, int32_t n_text, int32_t H, int32_t d, size_t *bytes) {
    if (!bytes) return fail(RTR_EINVAL, "bytes is NULL");
    *bytes = 0;
    if (Tq < 0 || Tq > kMaxTokens) return fail(RTR_EINVAL, "Tq=%lld out of range [0, 2^30]", (long long)Tq);
    if (n_text < 1) return fail(RTR_EINVAL, "n_text=%d must be >= 1", n_text);
    if (H < 1) return fail(RTR_EINVAL, "H=%d must be >= 1", H);
    if (d != 128) return fail(RTR_EUNSUPPORTED, "backward head dim %d not supported (128)", d);
    if (const hipError_t e = rtr::attention_cross_bwd_workspace_bytes(Tq, n_text, H, bytes)) return hip_fail(e, "workspace size");
    return ok();
}

int rtr_attn_cross_bwd(const rtr_text_cache *tc, const void *q, const void *o, const float *lse,
                       const void *d_o, int64_t Tq, void *dq, void *dk_text, void *dv_text, float scale,
                       void *workspace, size_t workspace_bytes, rtr_stream stream) {
    if (!tc) return fail(RTR_EINVAL, "cache handle is NULL");
    if (Tq < 0 || Tq > kMaxTokens) return fail(RTR_EINVAL, "Tq=%lld out of range [0, 2^30]", (long long)Tq);
    if (tc->dt != RTR_BF16) return fail(RTR_EUNSUPPORTED, "backward supports bf16 only");
    if (tc->d != 128) return fail(RTR_EUNSUPPORTED, "backward head dim %d not supported (128)", tc->d);
    if (int rc = check_scale(scale)) return rc;
    if (tc->n == 0) return fail(RTR_ESTATE, "the text cache holds no condition");
    if (Tq * tc->H * tc->d >= ((int64_t)1 << 31)) return fail(RTR_EUNSUPPORTED, "Tq * H * d must be below 2^31");
    if ((dk_text == nullptr) != (dv_text == nullptr))
        return fail(RTR_EINVAL, "dk_text and dv_text must both be NULL or both non-NULL");
    if (Tq == 0) return ok();
    const void *in[4] = {q, o, lse, d_o};
    for (const void *x : in)
        if (!x) return fail(RTR_EINVAL, "q, o, lse and d_o must be non-NULL");
    if (!dq) return fail(RTR_EINVAL, "dq must be non-NULL");
    for (const void *x : {q, o, d_o, (const void *)dq, (const void *)dk_text, (const void *)dv_text})
        if (!aligned16(x)) return fail(RTR_EINVAL, "tensor pointers must be 16-byte aligned");
    if (((uintptr_t)lse & 3u) != 0) return fail(RTR_EINVAL, "lse must be 4-byte aligned");
    const int64_t tok = (int64_t)tc->H * tc->d * 2;
    const int64_t tb = Tq * tok, lb = Tq * tc->H * 4, nb = (int64_t)tc->n * tok, cap_b = (int64_t)tc->capacity * tok;
    void *out[3] = {dq, dk_text, dv_text};
    const int64_t out_sz[3] = {tb, dk_text ? nb : 0, dv_text ? nb : 0};
    const void *src[6] = {q, o, lse, d_o, tc->k_buf, tc->v_buf};
    const int64_t src_sz[6] = {tb, tb, lb, tb, cap_b, cap_b};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(out[i], out_sz[i], src[j], src_sz[j])) return fail(RTR_EINVAL, "an output overlaps an input or the cache");
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(out[i], out_sz[i], out[j], out_sz[j])) return fail(RTR_EINVAL, "outputs overlap");
    }
    size_t need = 0;
    if (const hipError_t e = dk_text ? rtr::attention_cross_bwd_workspace_bytes(Tq, tc->n, tc->H, &need)
                                     : rtr::attention_bwd_workspace_bytes(Tq, tc->H, &need))
        return hip_fail(e, "workspace size");
    if (!workspace) return fail(RTR_EINVAL, "workspace is NULL (%zu bytes needed)", need);
    if (((uintptr_t)workspace & 255u) != 0) return fail(RTR_EINVAL, "workspace must be 256-byte aligned");
    if (workspace_bytes < need) return fail(RTR_EINVAL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    for (int j = 0; j < 6; ++j)
        if (overlaps(workspace, (int64_t)need, src[j], src_sz[j])) return fail(RTR_EINVAL, "workspace overlaps an input or the cache");
    for (int i = 0; i < 3; ++i)
        if (overlaps(workspace, (int64_t)need, out[i], out_sz[i])) return fail(RTR_EINVAL, "workspace overlaps an output");

    // The text tokens are the only keys, all seen by every query row: one
    // key segment that is all prefix, no keys of the rows' own.
    rtr::BwdProblem p;
    p.q = q;
    p.o = o;
    p.dout = d_o;
    p.lse = lse;
    p.dq = dq;
    p.T = Tq;
    p.tokens_per_frame = Tq;
    p.H = tc->H;
    p.scale = resolve_scale(scale, tc->d);
    p.ws = workspace;
    p.kseg[0] = tc->k_buf;
    p.vseg[0] = tc->v_buf;
    p.nseg = 1;
    p.seg_len = tc->n;
    p.prefix = tc->n;
    p.cross = true;
    p.dk_prefix = dk_text;
    p.dv_prefix = dv_text;
    if (const hipError_t e = rtr::launch_attention_bwd(p, (hipStream_t)stream)) return hip_fail(e, "backward launch");
    return ok();
}

int rtr_attn_cross(const rtr_text_cache *tc, const void *q, void *o, float *lse, int64_t Tq,
                   rtr_dtype out_dtype, float scale, void *workspace, size_t workspace_bytes,
                   rtr_stream stream) {
    if (!tc) return fail(RTR_EINVAL, "cache handle is NULL");
    if (Tq < 0 || Tq > kMaxTokens) return fail(RTR_EINVAL, "Tq=%lld out of range [0, 2^30]", (long long)Tq);
    if (!valid_dtype(out_dtype)) return fail(RTR_EINVAL, "unknown dtype");
    if (tc->dt == RTR_F32 && out_dtype != RTR_F32)
        return fail(RTR_EUNSUPPORTED, "float32 cache needs float32 output");
    if (int rc = check_scale(scale)) return rc;
    if (tc->n == 0) return fail(RTR_ESTATE, "the text cache holds no condition");
    if (Tq == 0) return ok();
    if (!q || !o) return fail(RTR_EINVAL, "q and o must be non-NULL");
    if (!aligned16(q) || !aligned16(o) || !aligned16(lse))
        return fail(RTR_EINVAL, "device pointers must be 16-byte aligned");
    const int64_t tok_in = (int64_t)tc->H * tc->d * esize(tc->dt);
    const int64_t in_b = Tq * tok_in, cap_b = tok_in * tc->capacity;
    const int64_t out_b = Tq * tc->H * tc->d * esize(out_dtype), lse_b = Tq * tc->H * 4;
    const void *ins[3] = {q, tc->k_buf, tc->v_buf};
    const int64_t in_sz[3] = {in_b, cap_b, cap_b};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(o, out_b, ins[i], in_sz[i])) return fail(RTR_EINVAL, "o overlaps q or the cache");
        if (overlaps(lse, lse_b, ins[i], in_sz[i])) return fail(RTR_EINVAL, "lse overlaps q or the cache");
    }
    if (overlaps(lse, lse_b, o, out_b)) return fail(RTR_EINVAL, "lse overlaps o");
    void *ws = nullptr;
    {
        const void *bufs[5] = {q, tc->k_buf, tc->v_buf, o, lse};
        const int64_t sizes[5] = {in_b, cap_b, cap_b, out_b, lse ? lse_b : 0};
        if (int rc = check_workspace(workspace, workspace_bytes, tc->d, tc->dt, bufs, sizes, 5, &ws)) return rc;
    }
    // Every query sees every text token: one key segment, all of it a prefix
    // that no frame limit cuts.
    rtr::AttnProblem p;
    p.ws = ws;
    p.q = q;
    p.o = o;
    p.lse = lse;
    p.kseg[0] = tc->k_buf;
    p.vseg[0] = tc->v_buf;
    p.nseg = 1;
    p.seg_len = tc->n;
    p.Tq = Tq;
    p.Tk = tc->n;
    p.prefix = tc->n;
    p.tokens_per_frame = Tq;
    p.H = tc->H;
    p.d = tc->d;
    p.scale = resolve_scale(scale, tc->d);
    p.in_dtype = tc->dt;
    p.out_dtype = out_dtype;
    const hipError_t e = rtr::launch_attention(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    return ok();
}

int rtr_kv_set_ref_rope(rtr_kv_cache *kv, void *k_ref_view, int32_t rope_pairs, float rope_base,
                        int64_t position_offset) {
    if (int rc = check_cache(kv)) return rc;
    if (!k_ref_view) {
        kv->k_ref_view = nullptr;
        kv->view_valid = false;
        return ok();
    }
    if (kv->R_cap < 1) return fail(RTR_ESTATE, "cache was created without reference capacity");
    if (rope_pairs < 1 || rope_pairs > kv->d / 2)
        return fail(RTR_EINVAL, "rope_pairs=%d outside [1, %d]", rope_pairs, kv->d / 2);
    if (!(rope_base > 1.0f) || std::isinf(rope_base)) return fail(RTR_EINVAL, "rope_base must be finite and > 1");
    if (position_offset < 0 || position_offset > kMaxTokens) return fail(RTR_EINVAL, "position_offset out of range");
    if (!aligned16(k_ref_view)) return fail(RTR_EINVAL, "k_ref_view must be 16-byte aligned");
    const int64_t fb = frame_bytes(kv);
    const void *bufs[4] = {kv->k_ring, kv->v_ring, kv->k_ref, kv->v_ref};
    const int64_t sizes[4] = {fb * kv->N, fb * kv->N, fb * kv->R_cap, fb * kv->R_cap};
    for (int i = 0; i < 4; ++i)
        if (overlaps(k_ref_view, fb * kv->R_cap, bufs[i], sizes[i]))
            return fail(RTR_EINVAL, "k_ref_view overlaps a cache buffer");
    kv->k_ref_view = k_ref_view;
    kv->rope_pairs = rope_pairs;
    kv->rope_base = rope_base;
    kv->pos_offset = position_offset;
    kv->view_valid = false;
    return ok();
}

int rtr_clock_sample(uint64_t *ticks, int64_t span_ticks, rtr_stream stream) {
    if (!ticks || ((uintptr_t)ticks & 7u) != 0) return fail(RTR_EINVAL, "ticks must be a non-NULL 8-byte aligned device pointer");
    if (span_ticks < 1 || span_ticks > 1000000) return fail(RTR_EINVAL, "span_ticks=%lld outside [1, 1e6]", (long long)span_ticks);
    if (const hipError_t e = rtr::launch_clock_probe((unsigned long long *)ticks, span_ticks, (hipStream_t)stream))
        return hip_fail(e, "clock probe launch");
    return ok();
}

int rtr_kv_get_state(const rtr_kv_cache *kv, rtr_kv_state *out) {
    if (int rc = check_cache(kv)) return rc;
    if (!out) return fail(RTR_EINVAL, "out is NULL");
    std::memset(out, 0, sizeof *out);
    out->window_frames = kv->W;
    out->ring_slots = kv->N;
    out->count = kv->count;
    out->head = kv->head;
    out->ref_frames = kv->ref_frames;
    out->ref_generation = kv->ref_gen;
    out->next_frame_id = kv->next_id;
    for (int p = 0; p < RTR_MAX_WINDOW; ++p) {
        out->slot[p] = -1;
        out->frame_id[p] = -1;
    }
    for (int p = 0; p < kv->count; ++p) {
        const int s = (kv->head + p) % kv->N;
        out->slot[p] = s;
        out->frame_id[p] = kv->slot_frame_id[s];
    }
    return ok();
}

int rtr_kv_set_state(rtr_kv_cache *kv, const rtr_kv_state *in) {
    if (int rc = check_cache(kv)) return rc;
    if (!in) return fail(RTR_EINVAL, "in is NULL");
    if (in->window_frames != kv->W) return fail(RTR_ESTATE, "snapshot window %d != cache window %d", in->window_frames, kv->W);
    if (in->ring_slots != kv->N)
        return fail(RTR_ESTATE, "snapshot ring slots %d != cache ring slots %d", in->ring_slots, kv->N);
    if (in->count < 0 || in->count > kv->W) return fail(RTR_ESTATE, "count out of range");
    if (kv->N > 0 ? (in->head < 0 || in->head >= kv->N) : in->head != 0) return fail(RTR_ESTATE, "head out of range");
    if (in->ref_frames < 0 || in->ref_frames > kv->R_cap) return fail(RTR_ESTATE, "ref_frames out of range");
    if (in->ref_generation < 0 || in->next_frame_id < 0) return fail(RTR_ESTATE, "negative counters");
    int64_t prev = -1;
    for (int p = 0; p < in->count; ++p) {
        if (in->slot[p] != (in->head + p) % kv->N) return fail(RTR_ESTATE, "slot list is not a ring from head");
        if (in->frame_id[p] <= prev || in->frame_id[p] >= in->next_frame_id)
            return fail(RTR_ESTATE, "frame ids must increase and stay below next_frame_id");
        prev = in->frame_id[p];
    }
    kv->count = in->count;
    kv->head = in->head;
    kv->ref_frames = in->ref_frames;
    kv->ref_gen = in->ref_generation;
    kv->next_id = in->next_frame_id;
    for (auto &x : kv->slot_frame_id) x = -1;
    for (int p = 0; p < in->count; ++p) kv->slot_frame_id[in->slot[p]] = in->frame_id[p];
    kv->view_valid = false;  // the restored reference may differ: rotate it again
    return ok();
}

}  // extern "C"
