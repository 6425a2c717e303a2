// Frame copies for the rolling KV ring (append / evict) and the anchored
// reference slot (RTR-DiT notes, "DiT as Real-Time Rerenderer ...", Key
// Designs 4).  The ring metadata (which frame goes to which slot) is decided on
// the host; this kernel only moves whole [k, H, d] frames.  It is bound by HBM
// bandwidth: every byte is read once and written once with 16-byte accesses
// that are contiguous across the workgroup, and each thread keeps four loads in
// flight before its stores.

#include "rtr_internal.h"

namespace rtr {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct CopyArgs {
    const u32x4 *src[kMaxCopies];
    u32x4 *dst[kMaxCopies];
    int64_t n16;  // 16-byte units per copy
};

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void frame_copy(const CopyArgs a) {
    const int job = blockIdx.y;
    const u32x4 *__restrict__ s = a.src[job];
    u32x4 *__restrict__ d = a.dst[job];
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + u * kThreads;
        if (i < a.n16) v[u] = s[i];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + u * kThreads;
        if (i < a.n16) d[i] = v[u];
    }
}

}  // namespace

hipError_t launch_frame_copies(const CopyJobs &jobs, hipStream_t stream) {
    if (jobs.n <= 0 || jobs.bytes <= 0) return hipSuccess;
    CopyArgs a{};
    for (int i = 0; i < jobs.n; ++i) {
        a.src[i] = (const u32x4 *)jobs.src[i];
        a.dst[i] = (u32x4 *)jobs.dst[i];
    }
    a.n16 = jobs.bytes / 16;
    const int64_t per_block = kThreads * kUnroll;
    const dim3 grid((unsigned)((a.n16 + per_block - 1) / per_block), (unsigned)jobs.n);
    hipLaunchKernelGGL(frame_copy, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rtr
