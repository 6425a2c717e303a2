// Frame copies for the rolling KV ring (append / evict) and the anchored
// reference slot (RTR-DiT notes, "DiT as Real-Time Rerenderer ...", Key
// Designs 4).  The ring metadata (which frame goes to which slot) is decided on
// the host; this kernel only moves whole [k, H, d] frames.  It is bound by HBM
// bandwidth: every byte is read once and written once with 16-byte accesses
// that are contiguous across the workgroup, and each thread keeps four loads in
// flight before its stores.

#include <cmath>

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

// Temporal rotary re-encoding of the anchored reference's K (position-aware
// cache): element pairs (2i, 2i+1), i < pairs, of every head row rotated by
// the angle whose cosine and sine the host computed for this shift; the other
// elements are copied.  One thread per 8 elements (16 bytes of bf16).
struct RotateArgs {
    const uint16_t *src;
    uint16_t *dst;
    int64_t n8;      // 8-element groups in all
    int32_t d8;      // 8-element groups per head row
    int32_t pairs;
    float cs[64], sn[64];
};

__global__ __launch_bounds__(kThreads) void ref_rotate_bf16(const RotateArgs a) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= a.n8) return;
    const u32x4 v = ((const u32x4 *)a.src)[i];
    const int p0 = (int)(i % a.d8) * 4;  // first pair of this group
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int p = p0 + w;
        if (p < a.pairs) {
            const float x0 = __uint_as_float(v[w] << 16), x1 = __uint_as_float(v[w] & 0xFFFF0000u);
            const float y0 = x0 * a.cs[p] - x1 * a.sn[p], y1 = x0 * a.sn[p] + x1 * a.cs[p];
            typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
            o[w] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y0, (__bf16)y1});
        } else {
            o[w] = v[w];
        }
    }
    ((u32x4 *)a.dst)[i] = o;
}

__global__ __launch_bounds__(kThreads) void ref_rotate_f32(const RotateArgs a) {
    // float32 cache: one thread per 4 elements (two pairs), n8 counts them.
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= a.n8) return;
    const u32x4 v = ((const u32x4 *)a.src)[i];
    const int p0 = (int)(i % a.d8) * 2;
    u32x4 o = v;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const int p = p0 + w;
        if (p < a.pairs) {
            const float x0 = __uint_as_float(v[2 * w]), x1 = __uint_as_float(v[2 * w + 1]);
            o[2 * w] = __float_as_uint(x0 * a.cs[p] - x1 * a.sn[p]);
            o[2 * w + 1] = __float_as_uint(x0 * a.sn[p] + x1 * a.cs[p]);
        }
    }
    ((u32x4 *)a.dst)[i] = o;
}

// Clock probe: one lane reads the shader-clock counter (s_memtime) and the
// constant 100 MHz counter (s_memrealtime) until `span` ticks of the latter
// have passed (at most 2^22 reads), and stores both differences.  Their ratio
// times 100 MHz is the shader clock over that interval.
__global__ __launch_bounds__(64) void clock_probe(unsigned long long *out, unsigned long long span) {
    if (threadIdx.x != 0) return;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long t1 = t0, r1 = r0;
    for (int i = 0; i < (1 << 22) && r1 - r0 < span; ++i) {
        t1 = __builtin_amdgcn_s_memtime();
        r1 = __builtin_amdgcn_s_memrealtime();
    }
    out[0] = t1 - t0;
    out[1] = r1 - r0;
}

}  // namespace

hipError_t launch_ref_rotate(const RotateJob &j, hipStream_t stream) {
    if (j.rows <= 0) return hipSuccess;
    RotateArgs a{};
    a.src = (const uint16_t *)j.src;
    a.dst = (uint16_t *)j.dst;
    a.pairs = j.pairs;
    const double two_pi = 6.283185307179586;
    for (int p = 0; p < j.pairs && p < 64; ++p) {
        // angle = shift * base^(-p / pairs), reduced in double before the float cast
        double ang = (double)j.shift * std::pow((double)j.base, -(double)p / j.pairs);
        ang = std::fmod(ang, two_pi);
        a.cs[p] = (float)std::cos(ang);
        a.sn[p] = (float)std::sin(ang);
    }
    const int per16 = j.dt == RTR_BF16 ? 8 : 4;  // elements per 16-byte group
    a.d8 = j.d / per16;
    a.n8 = j.rows * a.d8;
    const dim3 grid((unsigned)((a.n8 + kThreads - 1) / kThreads));
    if (j.dt == RTR_BF16)
        hipLaunchKernelGGL(ref_rotate_bf16, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(ref_rotate_f32, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

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

hipError_t launch_clock_probe(unsigned long long *out, int64_t span_ticks, hipStream_t stream) {
    hipLaunchKernelGGL(clock_probe, dim3(1), dim3(64), 0, stream, out, (unsigned long long)span_ticks);
    return hipGetLastError();
}

}  // namespace rtr
