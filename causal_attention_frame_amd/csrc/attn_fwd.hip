// Frame-block-causal attention forward for gfx950 (MI355X / CDNA4).
//
// Computes Attn(Q,K,V) = softmax(Q K^T * scale + M) V with the frame mask of
// the RTR-DiT notes ("DiT as Real-Time Rerenderer ...", Key Designs 2, Attn
// equation): query i sees key j iff floor(j/k) <= floor(i/k), generalised to a
// streaming call by `prefix` cached keys that every query sees (Key Designs 4).
// For one query row the visible keys are exactly [0, lim(i)) with
//   lim(i) = min(prefix + (floor(i/k) + 1) * k, Tk),
// so the mask is a per-row key limit, and whole key tiles beyond a
// workgroup's largest limit are never loaded.
//
// bf16 kernel (the hot path): one workgroup = 4 waves x 32 query rows of one
// head.  Per 64-key tile, K and V are staged through LDS from coalesced 16-byte
// global loads (prefetched into registers one tile ahead), then per wave:
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, K from LDS (A), Q^T held in
//                    registers for the whole kernel (B), fp32 accumulate;
//   online softmax   each lane owns one query column and 16 of every 32 keys,
//                    so the row max needs one cross-lane step (lane ^ 32);
//                    exp2 with scale*log2(e) folded into one FMA; P -> bf16 RNE;
//   O^T += V^T P^T   P^T comes straight out of the S^T accumulator registers
//                    (no shuffles) because V^T is written to LDS with its keys
//                    permuted inside each 16-key group to match the MFMA
//                    accumulator row order.
// The O^T accumulator puts one query per lane, so the softmax rescale is one
// scalar per lane.
//
// fp32 kernel: a plain VALU path for float32 inputs (one query row per
// thread), used where float32 accuracy is required; not tuned.

#include <cmath>
#include <type_traits>

#include "rtr_internal.h"

namespace rtr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

struct KArgs {
    const void *q;
    void *o;
    float *lse;
    const void *kseg[kMaxKeyFrames];
    const void *vseg[kMaxKeyFrames];
    int32_t nseg;        // segments in the table
    int32_t seg_len;     // keys per segment (all keys when there is one segment)
    float inv_seg_len;   // 1 / seg_len, for the segment lookup
    int32_t Tq, Tk, kpf, prefix;
    int64_t ld;          // row stride in elements (H * d)
    int32_t nqb, nwg;    // query blocks per head, workgroups in the grid
    float c;             // scale * log2(e)
    float scale;
    int32_t out_f32;
};

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.
// Give every XCD one contiguous range of work items so the query blocks of one
// head (which read the same K/V) share an L2; inside a head, the latest (most
// keys) query block goes first.
__device__ inline void map_block(int b, int nwg, int nqb, int &head, int &qb) {
    const int x = b & 7, i = b >> 3;
    const int q8 = nwg >> 3, r8 = nwg & 7;
    const int w = x * q8 + (x < r8 ? x : r8) + i;
    head = w / nqb;
    qb = nqb - 1 - (w - head * nqb);
}

__device__ inline int key_limit(int i, const KArgs &a) {
    const int f = i / a.kpf;
    const long lim = (long)a.prefix + (long)(f + 1) * a.kpf;
    return lim < a.Tk ? (int)lim : a.Tk;
}

// Segment holding key j (exact: the float estimate is corrected by one step).
__device__ inline int seg_of(int j, const KArgs &a) {
    int f = (int)((float)j * a.inv_seg_len);
    const int rem = j - f * a.seg_len;
    if (rem < 0) --f;
    else if (rem >= a.seg_len) ++f;
    return f;
}

template <bool SEG>
__device__ inline long key_offset(int j, const KArgs &a, int &f) {
    if (SEG) {
        f = seg_of(j, a);
        return (long)(j - f * a.seg_len) * a.ld;
    }
    f = 0;
    return (long)j * a.ld;
}

// Value of the same register in lane (lane ^ 32), combined with this lane's
// by max or sum: v_permlane32_swap exchanges the two 32-lane halves in place.
__device__ inline float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(1))) const u32x4 global_u32x4;

// 16-byte load through a global (not flat) address.
__device__ inline u32x4 gload16(const uint16_t *p) { return *(const global_u32x4 *)p; }

// Key addressing modes of the bf16 kernel.
enum SegMode : int {
    kContiguous = 0,  // one segment holds every key
    kSegAligned = 1,  // frame segments whose length is a multiple of 4 keys
    kSegGeneric = 2,  // frame segments of any length
};

// ---------------------------------------------------------------------------
// bf16 inputs, MFMA path.
// ---------------------------------------------------------------------------

// Online-softmax rescaling threshold in log2 units.  A row's reference max m is
// raised (and its O and l rescaled) only when a tile's row max exceeds m by
// more than this, so P = exp2((s - m) * scale * log2 e) < 2^8.  The softmax is
// unchanged (O and l share the reference); only rounding differs, and the
// O/l rescale, which touches every accumulator register, runs a few times per
// row instead of once per tile.
constexpr float kRescaleLog2 = 8.0f;

template <int D, int SEGMODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(const KArgs a) {
    constexpr bool SEG = SEGMODE != kContiguous;
    constexpr int BM = 128;         // query rows per workgroup (4 waves x 32)
    constexpr int BN = 64;          // keys per tile
    constexpr int KP = D + 8;       // LDS pitch of a K row (elements)
    constexpr int VP = BN + 8;      // LDS pitch of a V^T row (elements)
    constexpr int DC = D / 8;       // 16-byte chunks per row
    constexpr int NS = D / 16;      // MFMA k-steps over d
    constexpr int NT = D / 32;      // 32-wide column blocks of O^T
    constexpr int ITEMS = (BN / 4) * DC;  // loader items: 4 keys x 16 bytes
    static_assert(ITEMS <= 256, "tile loader needs at most one item per thread");
    static_assert(BN == 64, "the V^T swizzle assumes 8 blocks of 8 keys per row");

    // Double-buffered K and V^T tiles: tile t lives in buffer t & 1.
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[2][D * VP];
    __shared__ const uint16_t *sSegK[SEG ? kMaxKeyFrames : 1];
    __shared__ const uint16_t *sSegV[SEG ? kMaxKeyFrames : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, g = lane >> 5;

    int head, qb;
    map_block(blockIdx.x, a.nwg, a.nqb, head, qb);
    const int q0 = qb * BM;
    const long hoff = (long)head * D;

    const int qi = q0 + wave * 32 + n;
    const bool qvalid = qi < a.Tq;
    const int qc = qvalid ? qi : a.Tq - 1;
    const int lim = key_limit(qc, a);
    const int lim_wg_lo = key_limit(q0, a);
    const int lim_wg = key_limit(min(q0 + BM - 1, a.Tq - 1), a);
    const int wlim_hi = key_limit(min(q0 + wave * 32 + 31, a.Tq - 1), a);

    if (SEG) {
        for (int f = tid; f < a.nseg; f += 256) {
            sSegK[f] = (const uint16_t *)a.kseg[f];
            sSegV[f] = (const uint16_t *)a.vseg[f];
        }
    }

    // Q^T as the B operand: lane (n, g) holds q[qi][16 s + 8 g .. + 7].
    bf16x8 qf[NS];
    {
        const uint16_t *qrow = (const uint16_t *)a.q + (long)qc * a.ld + hoff;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            u32x4 raw = qvalid ? *(const u32x4 *)(qrow + 16 * s + 8 * g) : u32x4{0, 0, 0, 0};
            qf[s] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    if (SEG) __syncthreads();  // segment table visible to the loader

    // Tile loader: item (a4, ch) moves keys 4*a4 .. 4*a4+3, 16-byte chunk ch.
    const bool loader = tid < ITEMS;
    const int a4 = tid / DC, ch = tid % DC;
    u32x4 kreg[4], vreg[4];

    auto load_tile = [&](int j0) {
        const int jb = j0 + 4 * a4;
        if (SEGMODE == kSegGeneric) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = jb + r;
                if (loader && j < a.Tk) {
                    const int f = seg_of(j, a);
                    const long o = (long)(j - f * a.seg_len) * a.ld + hoff + ch * 8;
                    kreg[r] = gload16(sSegK[f] + o);
                    vreg[r] = gload16(sSegV[f] + o);
                } else {
                    kreg[r] = u32x4{0, 0, 0, 0};
                    vreg[r] = u32x4{0, 0, 0, 0};
                }
            }
            return;
        }
        // The 4 rows jb .. jb+3 lie in one segment (segments are multiples of
        // 4 keys, jb is a multiple of 4).
        const uint16_t *kb, *vb;
        long o;
        if (SEGMODE == kSegAligned) {
            const int f = min(seg_of(jb, a), a.nseg - 1);
            kb = sSegK[f];
            vb = sSegV[f];
            o = (long)(jb - f * a.seg_len) * a.ld + hoff + ch * 8;
        } else {
            kb = (const uint16_t *)a.kseg[0];
            vb = (const uint16_t *)a.vseg[0];
            o = (long)jb * a.ld + hoff + ch * 8;
        }
        if (loader && jb + 3 < a.Tk) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                kreg[r] = gload16(kb + o + r * a.ld);
                vreg[r] = gload16(vb + o + r * a.ld);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (loader && jb + r < a.Tk) {
                    kreg[r] = gload16(kb + o + r * a.ld);
                    vreg[r] = gload16(vb + o + r * a.ld);
                } else {
                    kreg[r] = u32x4{0, 0, 0, 0};
                    vreg[r] = u32x4{0, 0, 0, 0};
                }
            }
        }
    };

    auto store_tile = [&](int buf) {
        if (!loader) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) *(u32x4 *)&sK[buf][(4 * a4 + r) * KP + ch * 8] = kreg[r];
        // V^T with keys permuted inside each 16-key group: key group a (4 keys)
        // goes to position ((a&1)<<3)|((a>>1)<<2), so that lane half g of the
        // MFMA B operand finds its 8 keys {4g..4g+3, 8+4g..8+4g+3} contiguous.
        // Each row's eight 8-key blocks are XOR-swizzled by (row / 8) mod 8 so
        // the 16 threads writing rows 8 apart spread over the LDS banks; reads
        // of 8 consecutive rows stay conflict-free through the row padding.
        const int a = a4 & 3;
        const int blk = ((a4 >> 2) * 2 + (a & 1)) ^ (ch & 7);
        const int pos = blk * 8 + (a >> 1) * 4;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int w = e >> 1, sh = (e & 1) * 16;
            const uint32_t x0 = (vreg[0][w] >> sh) & 0xffffu;
            const uint32_t x1 = (vreg[1][w] >> sh) & 0xffffu;
            const uint32_t x2 = (vreg[2][w] >> sh) & 0xffffu;
            const uint32_t x3 = (vreg[3][w] >> sh) & 0xffffu;
            *(u32x2 *)&sVt[buf][(ch * 8 + e) * VP + pos] = u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
        }
    };

    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
    float m = -INFINITY, l = 0.f;
    const float c = a.c;
    const float grow_thr = kRescaleLog2 / c;

    // One tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
    auto step = [&](auto masked, int it) {
        constexpr bool MASK = decltype(masked)::value;
        const int j0 = it * BN;
        const uint16_t *Kt = sK[it & 1];
        const uint16_t *Vt = sVt[it & 1];
        // lane holds query n and keys 32 kt + 8 (r/4) + 4 g + (r%4)
        f32x16 s[BN / 32];
#pragma unroll
        for (int kt = 0; kt < BN / 32; ++kt) {
            s[kt] = f32x16{};
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const u32x4 raw = *(const u32x4 *)&Kt[(32 * kt + n) * KP + 16 * st + 8 * g];
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, raw), qf[st], s[kt], 0, 0, 0);
            }
        }
        if (MASK) {
#pragma unroll
            for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = j0 + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (j >= lim) s[kt][r] = -INFINITY;
                }
        }
        float mx = s[0][0];
#pragma unroll
        for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
        mx = pair_max(mx);
        // The branch is taken by the whole wave when any row needs it, but
        // only rows that crossed the threshold change their reference (the
        // others multiply by exactly 1), so each row's result depends on its
        // own keys only.
        const bool grow = mx > m + grow_thr;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? fmaxf(m, mx) : m;
            const float alpha = grow ? __builtin_amdgcn_exp2f((m - m_new) * c) : 1.f;
            l *= alpha;
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] *= alpha;
            m = m_new;
        }
        const float mc = m * c;
        bf16x8 pf[BN / 16];
#pragma unroll
        for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -mc));
                l += p;
                pf[2 * kt + (r >> 3)][r & 7] = (__bf16)p;
            }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int st = 0; st < BN / 16; ++st) {
                const int row = 32 * t + n;
                const int blk = (2 * st + g) ^ ((row >> 3) & 7);
                const u32x4 raw = *(const u32x4 *)&Vt[row * VP + blk * 8];
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, raw), pf[st], acc[t], 0, 0, 0);
            }
    };

    const int ntiles = (lim_wg + BN - 1) / BN;
    const int nfull = min(ntiles, lim_wg_lo / BN);  // tiles visible to every row here
    load_tile(0);
    store_tile(0);
    if (ntiles > 1) load_tile(BN);
    __syncthreads();
    int it = 0;
    for (; it < nfull; ++it) {
        if (it + 1 < ntiles) store_tile((it + 1) & 1);
        if (it + 2 < ntiles) load_tile((it + 2) * BN);
        step(std::false_type{}, it);
        __syncthreads();
    }
    for (; it < ntiles; ++it) {
        if (it + 1 < ntiles) store_tile((it + 1) & 1);
        if (it + 2 < ntiles) load_tile((it + 2) * BN);
        if (it * BN < wlim_hi) step(std::true_type{}, it);  // wave-uniform
        __syncthreads();
    }

    const float lt = pair_sum(l);
    const float inv = 1.f / lt;
    if (qvalid) {
        const long obase = (long)qi * a.ld + hoff;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dcol = 32 * t + 8 * i + 4 * g;
                const float o0 = acc[t][4 * i + 0] * inv, o1 = acc[t][4 * i + 1] * inv;
                const float o2 = acc[t][4 * i + 2] * inv, o3 = acc[t][4 * i + 3] * inv;
                if (a.out_f32) {
                    *(f32x4 *)((float *)a.o + obase + dcol) = f32x4{o0, o1, o2, o3};
                } else {
                    const uint32_t b0 = __builtin_bit_cast(uint16_t, (__bf16)o0);
                    const uint32_t b1 = __builtin_bit_cast(uint16_t, (__bf16)o1);
                    const uint32_t b2 = __builtin_bit_cast(uint16_t, (__bf16)o2);
                    const uint32_t b3 = __builtin_bit_cast(uint16_t, (__bf16)o3);
                    *(u32x2 *)((uint16_t *)a.o + obase + dcol) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
                }
            }
        if (g == 0 && a.lse) a.lse[(long)head * a.Tq + qi] = m * a.scale + logf(lt);
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs, VALU path: one query row per thread, 32-key tiles in LDS.
// ---------------------------------------------------------------------------
template <int D, bool SEG>
__global__ __launch_bounds__(64) void attn_fwd_f32(const KArgs a) {
    constexpr int BM = 64, BN = 32, DC = D / 4;
    __shared__ __attribute__((aligned(16))) float sK[BN * D];
    __shared__ __attribute__((aligned(16))) float sV[BN * D];

    const int tid = threadIdx.x;
    int head, qb;
    map_block(blockIdx.x, a.nwg, a.nqb, head, qb);
    const int q0 = qb * BM;
    const long hoff = (long)head * D;
    const int qi = q0 + tid;
    const bool qvalid = qi < a.Tq;
    const int qc = qvalid ? qi : a.Tq - 1;
    const int lim = key_limit(qc, a);
    const int lim_wg = key_limit(min(q0 + BM - 1, a.Tq - 1), a);

    float q[D], acc[D];
    const float *qrow = (const float *)a.q + (long)qc * a.ld + hoff;
#pragma unroll
    for (int e = 0; e < D; ++e) {
        q[e] = qrow[e];
        acc[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const float c = a.c;

    for (int j0 = 0; j0 < lim_wg; j0 += BN) {
        __syncthreads();
        for (int item = tid; item < BN * DC; item += BM) {
            const int r = item / DC, cc = item % DC;
            const int j = j0 + r;
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (j < a.Tk) {
                int f;
                const long off = key_offset<SEG>(j, a, f) + hoff + cc * 4;
                kv = *(const f32x4 *)((const float *)a.kseg[f] + off);
                vv = *(const f32x4 *)((const float *)a.vseg[f] + off);
            }
            *(f32x4 *)&sK[r * D + cc * 4] = kv;
            *(f32x4 *)&sV[r * D + cc * 4] = vv;
        }
        __syncthreads();
        float s[BN];
        float mx = -INFINITY;
#pragma unroll 4
        for (int jj = 0; jj < BN; ++jj) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) dot = fmaf(q[e], sK[jj * D + e], dot);
            s[jj] = (j0 + jj < lim) ? dot : -INFINITY;
            mx = fmaxf(mx, s[jj]);
        }
        const float m_new = fmaxf(m, mx);
        const float alpha = (m == -INFINITY) ? 0.f : exp2f((m - m_new) * c);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] *= alpha;
        for (int jj = 0; jj < BN; ++jj) {
            const float p = (s[jj] == -INFINITY) ? 0.f : exp2f((s[jj] - m_new) * c);
            l += p;
#pragma unroll
            for (int e = 0; e < D; ++e) acc[e] = fmaf(p, sV[jj * D + e], acc[e]);
        }
    }
    if (qvalid) {
        const float inv = 1.f / l;
        float *orow = (float *)a.o + (long)qi * a.ld + hoff;
#pragma unroll
        for (int e = 0; e < D; e += 4)
            *(f32x4 *)(orow + e) = f32x4{acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv,
                                         acc[e + 3] * inv};
        if (a.lse) a.lse[(long)head * a.Tq + qi] = m * a.scale + logf(l);
    }
}

template <int D, bool SEG>
hipError_t launch_d(const KArgs &ka, const AttnProblem &p, hipStream_t stream) {
    KArgs k = ka;
    if (p.in_dtype == RTR_BF16) {
        k.nqb = (int)((p.Tq + 127) / 128);
        k.nwg = k.nqb * p.H;
        if (!SEG)
            hipLaunchKernelGGL((attn_fwd_bf16<D, kContiguous>), dim3(k.nwg), dim3(256), 0, stream, k);
        else if (k.seg_len % 4 == 0)
            hipLaunchKernelGGL((attn_fwd_bf16<D, kSegAligned>), dim3(k.nwg), dim3(256), 0, stream, k);
        else
            hipLaunchKernelGGL((attn_fwd_bf16<D, kSegGeneric>), dim3(k.nwg), dim3(256), 0, stream, k);
    } else {
        k.nqb = (int)((p.Tq + 63) / 64);
        k.nwg = k.nqb * p.H;
        hipLaunchKernelGGL((attn_fwd_f32<D, SEG>), dim3(k.nwg), dim3(64), 0, stream, k);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnProblem &p, hipStream_t stream) {
    KArgs k{};
    k.q = p.q;
    k.o = p.o;
    k.lse = p.lse;
    for (int f = 0; f < p.nseg; ++f) {
        k.kseg[f] = p.kseg[f];
        k.vseg[f] = p.vseg[f];
    }
    k.nseg = p.nseg;
    k.seg_len = (int32_t)p.seg_len;
    k.inv_seg_len = 1.0f / (float)p.seg_len;
    k.Tq = (int32_t)p.Tq;
    k.Tk = (int32_t)p.Tk;
    k.kpf = (int32_t)p.tokens_per_frame;
    k.prefix = (int32_t)p.prefix;
    k.ld = (int64_t)p.H * p.d;
    k.scale = p.scale;
    k.c = p.scale * kLog2e;
    k.out_f32 = p.out_dtype == RTR_F32;
    const bool seg = p.nseg > 1;
    if (p.d == 128) return seg ? launch_d<128, true>(k, p, stream) : launch_d<128, false>(k, p, stream);
    return seg ? launch_d<64, true>(k, p, stream) : launch_d<64, false>(k, p, stream);
}

}  // namespace rtr
