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
// Kernels:
//   attn_fwd_bf16_d128        bf16, head_dim 128 (the hot path): 8 waves x 32
//                             query rows, K/V tiles staged into an LDS ring by
//                             global-to-LDS DMA, PV one tile behind the softmax;
//   attn_fwd_bf16_d128_split  the same work cut into pieces spread over idle
//                             workgroups (caller workspace), plus
//   attn_combine_d128         the fixed-order merge of the pieces;
//   attn_fwd_bf16             bf16, head_dim 64: 4 waves x 32 query rows, 64-key
//                             tiles staged through registers, V^T written to
//                             LDS with the MFMA accumulator's key order;
//   attn_fwd_f32              float32 inputs: one query row per thread, plain
//                             VALU, used where float32 accuracy is required.
// Every bf16 kernel computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (Q^T in
// registers for the whole kernel), the softmax in fp32 with exp2 and the scale
// folded into one FMA, P rounded to bf16 (RNE), and O^T += V^T P^T.

#include <algorithm>
#include <atomic>
#include <mutex>
#include <climits>
#include <cmath>
#include <cstddef>
#include <type_traits>

#include "device_util.h"
#include "rtr_internal.h"

namespace rtr {
namespace {

using namespace dev;

struct KArgs {
    const void *q;
    void *o;
    float *lse;
    // Segment base pointers; entry nseg repeats entry nseg - 1, so that a
    // segment and its successor can be read as one pair.
    const void *kseg[kMaxKeyFrames + 1];
    const void *vseg[kMaxKeyFrames + 1];
    int32_t nseg;        // segments in the table
    int32_t seg_len;     // keys per segment (all keys when there is one segment)
    float inv_seg_len;   // 1 / seg_len, for the segment lookup
    int32_t Tq, Tk, kpf, prefix;
    int64_t ld;          // row stride in elements (H * d)
    int32_t nqb, nwg;    // query blocks per head, workgroups in the grid
    float c;             // scale * log2(e)
    float scale;
    int32_t out_f32;
    // Split launch of the head_dim-128 kernel (nprog > 0): workspace of
    // partial-result slots, workgroups in the grid, units (heads x query
    // blocks), the common cut of the mains, spare workgroups, tail pieces in
    // all and tiles per tail piece.
    float *ws;
    int32_t nprog;
    int32_t units;
    int32_t cut;
    int32_t nspare;
    int32_t tail_total;
    int32_t piece;
    // Overflow split (nxqb > 0, units beyond the workgroups): query blocks qb
    // < nxqb of every head have no main, all their tiles are tail pieces, and
    // every workgroup takes its share of the pieces after its main, which
    // covers a whole unit: workgroup b the pieces [pk[b], pk[b + 8]) (the end
    // of its XCD's range when b + 8 is past the grid).
    int32_t nxqb;
    int16_t pk[256];
    // Row groups of the plain head_dim-128 kernel (its GMAP instance, picked
    // by plan_rows): 32-row groups per head (GMAP 1), or groups per frame,
    // frames and blocks per frame pair (GMAP 2).
    int32_t nwr;
    int32_t wpf, nframes, w1;
};

__host__ __device__ inline int key_limit(int i, const KArgs &a) {
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

// Key addressing modes of the bf16 kernel.
enum SegMode : int {
    kContiguous = 0,  // one segment holds every key
    kSegAligned = 1,  // frame segments long enough for the kernel's fast path
                      // (>= 4 keys and a multiple of 4 for the 64-query-block
                      // kernel; >= 32 keys for the head_dim-128 kernel)
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

    __shared__ int sMap[2];
    int head, qb;
    xcd_order_shared(blockIdx.x, a.nwg, a.nqb, head, qb, sMap);
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
// bf16 inputs, head_dim 128: 8 waves x 32 query rows, K/V staged by LDS DMA.
// ---------------------------------------------------------------------------
// A workgroup is 8 waves x 32 query rows of one head, two waves per SIMD: at
// 256 registers a wave, one wave's softmax VALU issues while the other's MFMAs
// run (a single wave per SIMD issues a VALU op only every ~7 cycles, so its
// softmax, not the matrix cores, set the pace).  Keys advance in 32-key tiles
// held in a 5-stage LDS ring that global_load_lds fills three tiles ahead of
// the compute (16 bytes per lane go straight from global memory to LDS: no
// staging registers, no VALU).  Layout of a stage (row-major, 256 B per key
// row; K tiles in one region, V tiles in another):
//   K: the 16-byte chunks of row r are XOR-swizzled by r mod 16: a
//      ds_read_b128 serves 16 lanes (rows n..n+15 of the MFMA A operand) per
//      pass over the 64 banks, and the swizzle gives them 16 distinct chunks;
//   V: the 64-byte chunk quads of row r are XOR-swizzled by r mod 4 and the
//      tile is read with ds_read_b64_tr_b16, whose 16-lane transpose hands each
//      lane one d column over 4 keys -- the V^T A operand of the PV MFMA in the
//      key order of the S^T accumulator, with no transposed copy anywhere.  A
//      pass of that read serves 32 lanes, 4 key rows x 64 bytes; the swizzle
//      puts the 4 rows in 4 distinct 64-byte bank groups (a 32-byte pair
//      swizzle left rows r and r ^ 1 on the same banks, a 2-way conflict).
// Synchronisation: one s_barrier per tile, after each wave has waited for its
// own DMA of that tile (vmcnt), so later prefetches stay in flight.
//
// The DMA is issued from inline assembly.  The compiler models a
// global-to-LDS load as touching both the vector-memory and the LDS counters
// and, while one is in flight, turns every LDS wait into a full drain; issued
// this way it is invisible to that model, the fragment reads get exact
// lgkmcnt waits, and the kernel waits for the DMA itself (vmcnt, in order).

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// A zero key/value row: keys past the end of a ragged key range are loaded from it.
__device__ __attribute__((aligned(16))) const uint16_t kZeroRow[128] = {};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; the clobber is still honoured
// One DMA load from a per-lane 64-bit address.
__device__ inline void dma16_vaddr(const void *src, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(m0)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Segment base pointers kseg[f], kseg[f + 1], vseg[f], vseg[f + 1].
struct SegPtrs {
    uint64_t k0, k1, v0, v1;
};
// The pointers of segments f and f + 1 as plain scalar loads from the kernel
// arguments, which the compiler waits for where they are first used.
__device__ inline SegPtrs load_seg_ptrs_ahead(int f) {
    typedef __attribute__((address_space(4))) const uint64_t c_u64;
    typedef __attribute__((address_space(4))) const char c_char;
    c_char *ka = (c_char *)__builtin_amdgcn_kernarg_segment_ptr();
    const c_u64 *kp = (const c_u64 *)(ka + offsetof(KArgs, kseg));
    const c_u64 *vp = (const c_u64 *)(ka + offsetof(KArgs, vseg));
    return {kp[f], kp[f + 1], vp[f], vp[f + 1]};
}



// DMA addressing of the head_dim-128 kernel.
enum DmaMode : int {
    kDmaFast = 0,  // segments of >= 32 keys, a multiple of 4 (one segment = contiguous keys):
                   // every 4-row DMA group lies in one segment, wave-uniform base
    kDmaLane = 1,  // anything else: per-lane segment lookup, zero rows past the end
};

template <int MODE, int GMAP>
__global__ __launch_bounds__(512) void attn_fwd_bf16_d128(const KArgs a) {
    constexpr int D = 128, BM = 256, BN = 32, NS = D / 16, NT = D / 32;
    constexpr int NB = 1;  // 32-row query blocks per wave (8 waves)
    constexpr int TILE = BN * D;  // elements of one K or V tile
    constexpr int NSTG = 5;       // LDS ring depth
    constexpr bool FAST = MODE == kDmaFast;
    // Tile t lives in stage (t mod 5): K tiles in one region and V tiles in
    // another, so every fragment read is a per-lane base plus an immediate
    // offset below 64 KB.
    __shared__ __attribute__((aligned(16))) uint16_t sK[NSTG * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t sV[NSTG * TILE];
    // Each wave's 32 query rows on their way in (Q) and out (bf16 O).
    __shared__ __attribute__((aligned(16))) uint16_t sQ[BM * D];
    __shared__ const uint16_t *sSegK[FAST ? 1 : kMaxKeyFrames];
    __shared__ const uint16_t *sSegV[FAST ? 1 : kMaxKeyFrames];
    __shared__ int sRedo;
    lds_u16 *const kbase = (lds_u16 *)sK;
    lds_u16 *const vbase = (lds_u16 *)sV;

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, g = lane >> 5;

    __shared__ int sMap[2];
    int head, qb;
    xcd_order_shared(blockIdx.x, a.nwg, a.nqb, head, qb, sMap);
    const long hoff = (long)head * D;
    // byte strides of the DMA addressing (a segment is below 2^31 bytes)
    const int32_t ld2 = (int32_t)(a.ld * 2), hoff2 = (int32_t)(hoff * 2);

    // Rows: each wave takes one group of up to 32 rows of its head.
    //  GMAP 0: blocks of 256 consecutive rows; wave w takes rows
    //          256 qb + 32 w .. + 31.
    //  GMAP 1: the head's nwr groups of 32 consecutive rows split into a light
    //          half [0, nlight) (fewer visible keys) and a heavy half; block
    //          qb's waves 0-3 take light groups 4 qb .. 4 qb + 3 and waves 4-7
    //          heavy groups nwr - 1 - 4 qb .. nwr - 4 - 4 qb.
    //  GMAP 2: groups follow the frames (wpf groups per frame, the last one
    //          ending with the frame, so that all rows of a group share one key
    //          limit); frame f is paired with frame F - 1 - f: w1 blocks per
    //          pair, waves 0-3 taking groups 4 q .. 4 q + 3 of the early frame
    //          and waves 4-7 the same groups of the late frame; with F odd the
    //          middle frame follows in blocks of 8 consecutive groups.
    // Waves w and w + 4 of a workgroup share a SIMD, so with GMAP 1 and 2 each
    // SIMD holds an early and a late group and blocks carry about equal work:
    // for a launch of one round, where blocks of consecutive rows leave the
    // compute units of the early frames idle while the last frame's blocks
    // finish.  GMAP 2 also keeps the groups of a block to one pair of frames,
    // so that no SIMD of a block still has two working waves after the
    // others have one (every step ends at a barrier of the whole block).  A
    // group outside its half or frame, or past the rows, has no rows here.
    const int nlight = (a.nwr + 1) >> 1;
    // first row and row count of wave w's group
    auto wave_rows = [&](int w, int &r0, int &nr) __attribute__((always_inline)) {
        r0 = 0;
        nr = 0;
        if constexpr (GMAP == 0) {
            r0 = BM * qb + 32 * w;
            nr = min(32, a.Tq - r0);
        } else if constexpr (GMAP == 1) {
            const int r = w < 4 ? 4 * qb + w : a.nwr - 1 - (4 * qb + w - 4);
            if (w < 4 ? r < nlight : r >= nlight) {
                r0 = 32 * r;
                nr = min(32, a.Tq - r0);
            }
        } else {
            // numbered from the last block, so that the dispatcher's
            // highest-index-first order starts the heaviest blocks (frame pair
            // 0) first and the light middle-frame blocks last
            const int np = a.nframes >> 1, b = a.nqb - 1 - qb;
            int f, j;
            if (b < np * a.w1) {
                const int fp = b / a.w1, q = b - fp * a.w1;
                f = w < 4 ? fp : a.nframes - 1 - fp;
                j = 4 * q + (w & 3);
            } else {
                f = np;
                j = 8 * (b - np * a.w1) + w;
            }
            if (j < a.wpf) {
                r0 = f * a.kpf + 32 * j;
                nr = min(min(32, a.kpf - 32 * j), a.Tq - r0);
            }
        }
    };
    int qrow0, nrows;  // this wave's first row and row count
    wave_rows(wave, qrow0, nrows);
    const bool wvalid = nrows > 0;

    int qi[NB], lim[NB];
    bool qv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        qi[b] = qrow0 + 32 * b + n;
        qv[b] = 32 * b + n < nrows;
        lim[b] = key_limit(qv[b] ? qi[b] : a.Tq - 1, a);
    }
    // Key limit of this wave's last valid row (limits grow with the row), 0
    // for a wave without valid rows: steps past it skip the wave's MFMAs and
    // softmax (it still loads its share of the tiles and meets the barriers).
    const int lim_wave = wvalid ? key_limit(qrow0 + nrows - 1, a) : 0;
    // The block's largest limit sets the steps every wave takes: that of the
    // last row of its highest group (limits grow with the row): wave 7's
    // group with GMAP 0, wave 4's with GMAP 1 and 2 (that of a middle-frame
    // block of GMAP 2 has wave 0's limit, as has a frame-pair block whose
    // late groups are empty), or the highest light group (GMAP 1).
    int lim_wg;
    if constexpr (GMAP == 0) {
        lim_wg = key_limit(min(BM * qb + BM - 1, a.Tq - 1), a);
    } else {
        int r0 = 0, nr = 0;
        if constexpr (GMAP == 1) {
            const int hr = a.nwr - 1 - 4 * qb;
            r0 = 32 * (hr >= nlight ? hr : min(4 * qb + 3, nlight - 1));
            nr = min(32, a.Tq - r0);
        } else {
            wave_rows(a.nqb - 1 - qb < (a.nframes >> 1) * a.w1 ? 4 : 0, r0, nr);
            // a frame pair whose late-frame groups lie past the rows (a
            // partial last frame) has the early frame's limit
            if (nr <= 0) wave_rows(0, r0, nr);
        }
        lim_wg = key_limit(nr > 0 ? r0 + nr - 1 : a.Tq - 1, a);
    }

    if (!FAST) {
        for (int f = tid; f < a.nseg; f += 512) {
            sSegK[f] = (const uint16_t *)a.kseg[f];
            sSegV[f] = (const uint16_t *)a.vseg[f];
        }
    }
    if (tid == 0) sRedo = 0;
    __syncthreads();

    // DMA: this wave fills tile rows 4 wave + lr of K and of V, lane (lr, pch)
    // the physical 16-byte chunk pch, fetching the logical chunk that the
    // swizzle puts there.
    const int lr = lane >> 4, pch = lane & 15;

    // Q^T B operands: lane (n, g) holds q[qi][16 s + 8 g .. + 7].  The wave's
    // rows first go to its part of sQ by DMA, whole 256-byte rows per
    // instruction (4 rows; a row's 16-byte chunks XOR-swizzled by row mod 16,
    // as for K), so that every request covers whole cache lines, where loading
    // the fragments directly would touch each line with eight requests of 32
    // bytes.  They land before key tile 0 (older DMAs); the first sweep reads
    // the fragments back.  Rows past Tq read the last row and are zeroed.
    bf16x8 qf[NB][NS];
    lds_u16 *const qw = (lds_u16 *)sQ + wave * 32 * D;
    if (wvalid) {
        const uint64_t qp = (uint64_t)((const uint16_t *)a.q + (long)qrow0 * a.ld + hoff);
        const uint64_t qbase = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)qp) |
                               ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(qp >> 32)) << 32);
        const int rmax = nrows - 1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 4 * j + lr;
            dma16(qbase, (uint32_t)(min(r, rmax) * ld2 + ((pch ^ (r & 15)) << 4)),
                  lds_addr(qw) + (uint32_t)(j * 4 * D * 2));
        }
    }
    int kch[1], vch[1];
    uint32_t kvo[1], vvo[1];  // per-lane byte offsets from the group's first row
#pragma unroll
    for (int i = 0; i < 1; ++i) {
        kch[i] = pch ^ (4 * (wave & 3) + lr);           // (row mod 16) = 4 (wave mod 4) + lr
        vch[i] = (((pch >> 2) ^ lr) << 2) | (pch & 3);  // (row mod 4) = lr
        kvo[i] = (uint32_t)(((long)lr * a.ld + kch[i] * 8) * 2);
        vvo[i] = (uint32_t)(((long)lr * a.ld + vch[i] * 8) * 2);
    }
    const uint32_t k_lds = lds_addr(kbase), v_lds = lds_addr(vbase);
    auto m0k = [&](int S, int i) __attribute__((always_inline)) { return k_lds + (uint32_t)((S * TILE + (4 * wave + 4 * i) * D) * 2); };
    auto m0v = [&](int S, int i) __attribute__((always_inline)) { return v_lds + (uint32_t)((S * TILE + (4 * wave + 4 * i) * D) * 2); };

    // DMA cursor of this wave's 4-row group (tiles are prefetched in order
    // within a sweep; wave-uniform): the group's row drow inside segment dseg
    // (a group never straddles two segments: segments hold a multiple of 4
    // keys).  prepare() turns it into the K and V addresses of the next tile's
    // group and moves it one tile on.  Past the last segment it wraps inside
    // the last one, so look-ahead tiles beyond the keys still read valid
    // (finite) rows, which the mask discards.  Steps call prepare() before
    // their barrier, where its scalar work overlaps the wait.
    // The segment pointers are loaded one tile ahead (nsp), so that their
    // latency is not waited for at the barrier.
    int drow = 0, dseg = 0;
    uint64_t dkp = 0, dvp = 0;
    SegPtrs nsp{};
    auto reset_cursor = [&]() __attribute__((always_inline)) {
        drow = 4 * wave;
        dseg = 0;
        if constexpr (FAST) nsp = load_seg_ptrs_ahead(0);
    };
    auto prepare = [&]() __attribute__((always_inline)) {
        if constexpr (FAST) {
            const uint64_t off = (uint64_t)(uint32_t)(drow * ld2 + hoff2);
            dkp = nsp.k0 + off;
            dvp = nsp.v0 + off;
            drow += BN;
            const bool cr = drow >= a.seg_len;
            drow = cr ? drow - a.seg_len : drow;
            dseg = cr ? min(dseg + 1, a.nseg - 1) : dseg;
            nsp = load_seg_ptrs_ahead(dseg);
        }
    };
    auto issue = [&](int tile, auto S) __attribute__((always_inline)) {
        constexpr int st = decltype(S)::value;
        if constexpr (FAST) {
            dma16x2(dkp, dvp, kvo[0], vvo[0], m0k(st, 0), m0v(st, 0));
        } else {
            const int j0 = tile * BN;
#pragma unroll
            for (int i = 0; i < 1; ++i) {
                const int j = j0 + 4 * wave + 4 * i + lr;
                const uint16_t *kp = kZeroRow + kch[i] * 8;
                const uint16_t *vp = kZeroRow + vch[i] * 8;
                if (j < a.Tk) {
                    const int f = seg_of(j, a);
                    const long o = (long)(j - f * a.seg_len) * a.ld + hoff;
                    kp = sSegK[f] + o + kch[i] * 8;
                    vp = sSegV[f] + o + vch[i] * 8;
                }
                dma16_vaddr(kp, m0k(st, i));
                dma16_vaddr(vp, m0v(st, i));
            }
        }
    };

    // Per-lane LDS pointers of the fragment reads in stage 0; the stage, the
    // upper half of d and the key steps are immediate offsets.
    const lds_u16 *kfp[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) kfp[s] = kbase + n * D + (((2 * s + g) ^ (n & 15)) << 3);
    const int G = lane >> 4, sl = lane & 15;
    const int vrow = 4 * (G >> 1) + (sl >> 2);  // + 16 key-step + 8 half
    const lds_u16 *vfp[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        vfp[t] = vbase + vrow * D + ((2 * (t ^ (sl >> 2)) + (G & 1)) << 4) + 4 * (sl & 3);

    // Softmax with a fixed per-row exponent reference (log2 units): P =
    // exp2(s * c - mref).  mref is the row max of the row's first key tile, so
    // P <= 1 there; later tiles may exceed it, which is harmless while the
    // running sum stays far from the fp32 range.  A row whose sum ends above
    // 2^64 (or overflows) is recomputed in a second pass with its exact row max
    // as reference.  The accumulators are therefore touched only by MFMAs inside
    // the key loop.  Each row's result depends on its own scores only.  The row
    // sum adds the bf16-rounded P that the PV product uses.
    f32x16 acc[NB][NT];
    float mref[NB] = {0.f}, l[NB] = {0.f}, mmax[NB] = {-INFINITY};
    const float c = a.c;

    // Every wave takes the block's ntiles + 1 steps (one barrier each); a wave
    // runs the unmasked steps up to its own first row's limit, so that a block
    // whose rows span two frames keeps the masked steps to the wave whose rows
    // do.
    const int ntiles = (lim_wg + BN - 1) / BN;
    const int nfull = lim_wave > 0 ? min(ntiles, key_limit(qrow0, a) / BN) : 0;

    // Fragment reads of one tile: K (A operand of S^T = K Q^T, 8 k-steps over d)
    // and V^T (A operand of O^T += V^T P^T, 4 column blocks x 2 key steps, two
    // transposed 8-byte reads each).
    auto read_k = [&](auto S, bf16x8 *kf) __attribute__((always_inline)) {
        constexpr int st = decltype(S)::value;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            kf[s] = __builtin_bit_cast(bf16x8, *(lds_u32x4 *)(kfp[s] + st * TILE));
    };
    auto read_v = [&](auto S, v4i16 (*vf)[2][2]) __attribute__((always_inline)) {
        constexpr int st = decltype(S)::value;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                vf[t][s][0] = lds_tr16(vfp[t] + st * TILE + (16 * s) * D);
                vf[t][s][1] = lds_tr16(vfp[t] + st * TILE + (16 * s + 8) * D);
            }
    };
    // S^T = K Q^T: lane holds query n of each block and keys 8 (r/4) + 4 g + (r%4).
    auto qk = [&](const bf16x8 *kf, f32x16 *s) __attribute__((always_inline)) {
        s[0] = f32x16{};
#pragma unroll
        for (int st = 0; st < NS; ++st) s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[0][st], s[0], 0, 0, 0);
    };
    auto apply_mask = [&](f32x16 *s, int tile) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (tile * BN + 8 * (r >> 2) + 4 * g + (r & 3) >= lim[b]) s[b][r] = -INFINITY;
    };
    auto rowmax = [&](const f32x16 &s) __attribute__((always_inline)) {
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        return pair_max(mx);
    };
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    auto softmax = [&](const f32x16 *s, bf16x8 (*pf)[2], const float *mr) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pf[b][h][j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[b][8 * h + j], c, -mr[b]));
                const bf16x8 &p8 = pf[b][h];
                l[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 0, 1), ones, l[b], false);
                l[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 2, 3), ones, l[b], false);
                l[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 4, 5), ones, l[b], false);
                l[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 6, 7), ones, l[b], false);
            }
    };
    // O^T += V^T P^T.
    auto pv = [&](v4i16 (*vf)[2][2], bf16x8 (*pf)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const bf16x8 v = __builtin_bit_cast(
                    bf16x8, (v8i16)__builtin_shufflevector(vf[t][st][0], vf[t][st][1], 0, 1, 2, 3, 4, 5, 6, 7));
                acc[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, pf[0][st], acc[0][t], 0, 0, 0);
            }
    };

    // Software pipeline over key tiles, PV one tile behind the softmax.  Step
    // t (stage s(t) = t mod 5): wait until this wave's DMA of tile t+1 has
    // landed (t+2 may still be in flight), barrier (every wave's DMA of t+1 has
    // landed; every wave is done with step t-1, so the stage of tile t-2 is
    // free), then in one basic block: the K(t+1) fragment reads; O += V(t-1)
    // P(t-1) from registers, each MFMA followed by the transposed reads of the
    // V(t) fragments that take over its A operand's registers (they feed the
    // PV of step t+1); then S(t+1) = K(t+1) Q^T; the VALU turns S(t) into P(t)
    // under both; last the prefetch of tile t+3 into the stage of tile t-2.
    // The step after the last tile only adds the last PV (its tile is past
    // every row's limit, so its P is 0).
    //
    // Masked steps: a row whose limit lies at or below the tile start takes an
    // infinite exponent reference (P = 0); the element-wise mask runs only when
    // some row's limit falls inside the tile, at most a few tiles per block.
    //
    // S and P live in two register sets each.  In the unmasked loop the steps
    // alternate them (parity PAR reads set PAR and writes set PAR ^ 1), so that
    // no step ends with a copy of the next tile's S and P into the current
    // ones, in groups of ten steps (five stages x two parities); the masked
    // tail (PAR 2) keeps set 0 current and copies, in groups of five, because
    // its exit tests after every step would keep both sets live.
    f32x16 sbuf[2][NB];
    bf16x8 pbuf[2][NB][2];
    v4i16 vcur[NT][2][2];  // V^T fragments of the tile whose PV runs next
    auto step = [&](int t, auto S, auto masked, auto maxonly, auto par) __attribute__((always_inline)) {
        constexpr int s0 = decltype(S)::value;
        constexpr bool MASK = decltype(masked)::value;
        constexpr bool MAXONLY = decltype(maxonly)::value;
        constexpr int PAR = decltype(par)::value;
        constexpr bool COPY = PAR == 2;
        f32x16 stmp[NB];
        bf16x8 ptmp[NB][2];
        f32x16 *const scur = sbuf[COPY ? 0 : PAR];
        f32x16 *const snext = COPY ? stmp : sbuf[PAR ^ 1];
        bf16x8 (*const pprev)[2] = pbuf[COPY ? 0 : PAR];
        bf16x8 (*const pf)[2] = COPY ? ptmp : pbuf[PAR ^ 1];
        prepare();  // DMA addresses of tile t + 3
        // this wave's DMA of tile t+1 has landed (t+2 may still be in flight);
        // after the barrier every wave's has, and every wave is done with
        // step t-1, so the stage of tile t-2 is free
        __builtin_amdgcn_s_waitcnt(wait_vm(2));
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        if (MASK && (t - 1) * BN >= lim_wave) {
            // nothing left for this wave: tiles t-1 and later lie past every
            // one of its rows' limits (only in the masked tail, so that the
            // unmasked steps stay one basic block)
            issue(t + 3, std::integral_constant<int, (s0 + 3) % NSTG>{});
            return;
        }
        float mr[NB] = {mref[0]};
        if (MASK) {
            const int t0 = t * BN;
            bool part = false;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                part = part || (lim[b] > t0 && lim[b] < t0 + BN);
                mr[b] = lim[b] <= t0 ? INFINITY : mref[b];
            }
            if (MAXONLY || __builtin_amdgcn_ballot_w64(part)) {
                asm volatile("");
                apply_mask(scur, t);
            }
        }
        bf16x8 kf[NS];
        read_k(std::integral_constant<int, (s0 + 1) % NSTG>{}, kf);
        __builtin_amdgcn_sched_barrier(0);  // the K reads go first
        if (MAXONLY) {
            qk(kf, snext);
#pragma unroll
            for (int b = 0; b < NB; ++b) mmax[b] = fmaxf(mmax[b], rowmax(scur[b]));
            issue(t + 3, std::integral_constant<int, (s0 + 3) % NSTG>{});
        } else {
            pv(vcur, pprev);
            read_v(std::integral_constant<int, s0>{}, vcur);
            softmax(scur, pf, mr);
            qk(kf, snext);
            issue(t + 3, std::integral_constant<int, (s0 + 3) % NSTG>{});
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
            if (COPY) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int h = 0; h < 2; ++h) pbuf[0][b][h] = ptmp[b][h];
            }
        }
        if (COPY) sbuf[0][0] = stmp[0];
    };
    auto sweep = [&](bool first_sweep, auto maxonly) __attribute__((always_inline)) {
        reset_cursor();
        prepare();
        issue(0, I0{});
        prepare();
        issue(1, I1{});
        prepare();
        issue(2, I2{});
        __builtin_amdgcn_s_waitcnt(wait_vm(4));  // tile 0 landed
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        if (lim_wave == 0) {
            // A wave without valid rows only loads its share of the tiles and
            // meets the barriers of the steps.
            auto idle = [&](int t, auto S) __attribute__((always_inline)) {
                constexpr int s0 = decltype(S)::value;
                prepare();
                __builtin_amdgcn_s_waitcnt(wait_vm(2));
                compiler_fence();
                __builtin_amdgcn_s_barrier();
                compiler_fence();
                issue(t + 3, std::integral_constant<int, (s0 + 3) % NSTG>{});
            };
#pragma unroll 1
            for (int base = 0; base <= ntiles; base += 5) {
                idle(base, I0{});
                if (base + 1 > ntiles) break;
                idle(base + 1, I1{});
                if (base + 2 > ntiles) break;
                idle(base + 2, I2{});
                if (base + 3 > ntiles) break;
                idle(base + 3, I3{});
                if (base + 4 > ntiles) break;
                idle(base + 4, I4{});
            }
            return;  // look-ahead tiles still in flight: see drain()
        }
        if (first_sweep) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const bf16x8 v = lds_b128(qw + n * D + (((2 * s + g) ^ (n & 15)) << 3));
                qf[0][s] = qv[0] ? v : bf16x8{};
            }
        }
        {
            bf16x8 kf[NS];
            read_k(I0{}, kf);
            qk(kf, sbuf[0]);
        }
        if (first_sweep) {
            if (0 >= nfull) apply_mask(sbuf[0], 0);
#pragma unroll
            for (int b = 0; b < NB; ++b) mref[b] = rowmax(sbuf[0][b]) * c;
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h) pbuf[0][b][h] = bf16x8{};
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int ss = 0; ss < 2; ++ss) vcur[tt][ss][0] = vcur[tt][ss][1] = v4i16{0, 0, 0, 0};
        // Groups of ten steps (static stages and parities): unmasked while the
        // whole group is visible to every row, masked from there on, up to the
        // step after the last tile (which only adds the last PV).
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        using PC = std::integral_constant<int, 2>;
        int base = 0;
        if constexpr (FAST) {
#pragma unroll 1
            for (; base + 10 <= nfull; base += 10) {
                step(base, I0{}, std::false_type{}, maxonly, P0{});
                step(base + 1, I1{}, std::false_type{}, maxonly, P1{});
                step(base + 2, I2{}, std::false_type{}, maxonly, P0{});
                step(base + 3, I3{}, std::false_type{}, maxonly, P1{});
                step(base + 4, I4{}, std::false_type{}, maxonly, P0{});
                step(base + 5, I0{}, std::false_type{}, maxonly, P1{});
                step(base + 6, I1{}, std::false_type{}, maxonly, P0{});
                step(base + 7, I2{}, std::false_type{}, maxonly, P1{});
                step(base + 8, I3{}, std::false_type{}, maxonly, P0{});
                step(base + 9, I4{}, std::false_type{}, maxonly, P1{});
            }
        } else {  // per-lane addressing: its extra registers leave no room for two sets
#pragma unroll 1
            for (; base + 5 <= nfull; base += 5) {
                step(base, I0{}, std::false_type{}, maxonly, PC{});
                step(base + 1, I1{}, std::false_type{}, maxonly, PC{});
                step(base + 2, I2{}, std::false_type{}, maxonly, PC{});
                step(base + 3, I3{}, std::false_type{}, maxonly, PC{});
                step(base + 4, I4{}, std::false_type{}, maxonly, PC{});
            }
        }
#pragma unroll 1
        for (; base <= ntiles; base += 5) {
            step(base, I0{}, std::true_type{}, maxonly, PC{});
            if (base + 1 > ntiles) break;
            step(base + 1, I1{}, std::true_type{}, maxonly, PC{});
            if (base + 2 > ntiles) break;
            step(base + 2, I2{}, std::true_type{}, maxonly, PC{});
            if (base + 3 > ntiles) break;
            step(base + 3, I3{}, std::true_type{}, maxonly, PC{});
            if (base + 4 > ntiles) break;
            step(base + 4, I4{}, std::true_type{}, maxonly, PC{});
        }
        // The look-ahead tiles past the last one may still be in flight here;
        // drain() waits for them before the stages are reused or the wave
        // ends, so that their latency overlaps the epilogue.
    };
    auto drain = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(wait_vm(0));
        compiler_fence();
    };

#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[b][t] = f32x16{};
    sweep(true, std::false_type{});

    // Rare second pass for rows whose sum left the safe range.
    const float kSafeSum = 18446744073709551616.f;  // 2^64
    bool redo[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) redo[b] = qv[b] && !(pair_sum(l[b]) <= kSafeSum);
    if (__builtin_amdgcn_ballot_w64(redo[0]) && lane == 0) sRedo = 1;
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(sRedo)) {
        asm volatile("");
        drain();
        sweep(false, std::true_type{});  // exact row maxima
        drain();
        __syncthreads();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (redo[b]) mref[b] = mmax[b] * c;
            l[b] = 0.f;
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[b][t] = f32x16{};
        }
        sweep(false, std::false_type{});
    }

    const float lt = pair_sum(l[0]);
    const float inv = 1.f / lt;
    if (a.out_f32) {
        if (qv[0]) {
            const long obase = (long)qi[0] * a.ld + hoff;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *(f32x4 *)((float *)a.o + obase + 32 * t + 8 * i + 4 * g) =
                        f32x4{acc[0][t][4 * i] * inv, acc[0][t][4 * i + 1] * inv, acc[0][t][4 * i + 2] * inv,
                              acc[0][t][4 * i + 3] * inv};
        }
    } else if (wvalid) {
        // bf16 O through the wave's part of sQ (its Q fragments were read in
        // the first sweep): written in the accumulator layout (row n, columns
        // 32 t + 8 i + 4 g .. + 3, chunks swizzled as for Q), then read back
        // and stored as whole 256-byte rows, 16 bytes per lane.
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(__attribute__((address_space(3))) u32x2 *)(qw + n * D + (((4 * t + i) ^ (n & 15)) << 3) + 4 * g) =
                    u32x2{pack_bf16x2(acc[0][t][4 * i] * inv, acc[0][t][4 * i + 1] * inv),
                          pack_bf16x2(acc[0][t][4 * i + 2] * inv, acc[0][t][4 * i + 3] * inv)};
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        compiler_fence();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 4 * j + lr;
            const u32x4 v = *(lds_u32x4 *)(qw + r * D + (pch << 3));
            if (r < nrows)
                *(u32x4 *)((uint16_t *)a.o + (long)(qrow0 + r) * a.ld + hoff + ((pch ^ (r & 15)) << 3)) = v;
        }
    }
    if (g == 0 && a.lse && qv[0]) a.lse[(long)head * a.Tq + qi[0]] = mref[0] / kLog2e + logf(lt);
    drain();
}

// Work decomposition of the head_dim-128 kernel.  A unit is one (head, query
// block of 256 rows), head-major (u = head * nqb + qb); it covers the key tiles
// [0, n(qb)), n(qb) the tiles up to the block's largest key limit.
//
// Plain launch (attn_fwd_bf16_d128 above): one workgroup per unit.
//
// Split launch (attn_fwd_bf16_d128_split below, with a workspace), for U units
// on G > U workgroups: every unit keeps one "main" workgroup, and the mains
// all walk the keys from tile 0 in step, so the query blocks of one head share
// each K/V tile through L2; but a main stops at a common cut T.  The tail [T,
// n) of a longer unit is cut into pieces of P tiles (unit-major order, piece k
// of K), and the S = G - U spare workgroups share them evenly by count (spare
// s: pieces [s K / S, (s + 1) K / S)) while the mains run.  T and P come from
// the host, which simulates this schedule for the problem's unit lengths and
// picks the shortest.  Pieces that are not whole units leave
// unnormalised partial results in the workspace: the main of unit u in slot u,
// tail piece k in slot U + k; the combine kernel merges each split unit's
// pieces in that fixed order.
constexpr int kD128BM = 256, kD128BN = 32;
constexpr int kMaxSplitUnits = 256;                       // units of a split launch
constexpr int kSlotFloats = kD128BM * 128 + 2 * kD128BM;  // partial O, reference, sum
static_assert(kSlotFloats * sizeof(float) == kSplitSlotBytes, "slot size");

__host__ __device__ inline int block_tiles(int qb, const KArgs &a) {
    const int last = min(qb * kD128BM + kD128BM - 1, a.Tq - 1);
    return (key_limit(last, a) + kD128BN - 1) / kD128BN;
}

// Tail pieces of unit u.
__host__ __device__ inline int unit_pieces(int u, const KArgs &a) {
    const int qb = u % a.nqb;
    if (a.nxqb > 0) return qb < a.nxqb ? (block_tiles(qb, a) + a.piece - 1) / a.piece : 0;
    const int r = block_tiles(qb, a) - a.cut;
    return r > 0 ? (r + a.piece - 1) / a.piece : 0;
}

// Units that can have tail pieces, in unit order: every unit, or with an
// overflow split the nxqb first query blocks of each head.
__host__ __device__ inline int piece_units(const KArgs &a) {
    return a.nxqb > 0 ? (a.units / a.nqb) * a.nxqb : a.units;
}
__host__ __device__ inline int piece_unit(int pu, const KArgs &a) {
    return a.nxqb > 0 ? (pu / a.nxqb) * a.nqb + pu % a.nxqb : pu;
}

// sPre[i] = tail pieces of piece units 0 .. i-1 (i = 0 .. piece_units), built
// by the first 256 threads of the workgroup, one unit each; every thread takes
// the barriers.
__device__ __forceinline__ void build_piece_prefix(const KArgs &a, int *sPre, int *sTmp) {
    const int tid = threadIdx.x;
    if (tid < 256) sTmp[tid] = tid < piece_units(a) ? unit_pieces(piece_unit(tid, a), a) : 0;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive scan
        const int v = (tid < 256 && tid >= off) ? sTmp[tid - off] : 0;
        __syncthreads();
        if (tid < 256) sTmp[tid] += v;
        __syncthreads();
    }
    if (tid < 256) sPre[tid + 1] = sTmp[tid];
    if (tid == 0) sPre[0] = 0;
    __syncthreads();
}

// Largest u with sPre[u] <= x (sPre non-decreasing).
__host__ __device__ inline int find_tail_unit(const int *sPre, int U, int x) {
    int lo = 0, hi = U;  // sPre[lo] <= x < sPre[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sPre[mid] <= x) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Role of workgroup b in a split launch.  Workgroup b runs on XCD b mod 8;
// each XCD gets a contiguous head-major run of units (so the mains of one head
// share that XCD's L2), and its remaining workgroups are spares.
__host__ __device__ inline void split_role(int b, const KArgs &a, int &unit, int &spare) {
    const int x = b & 7, i = b >> 3;
    unit = -1;
    spare = -1;
    if (a.nxqb > 0) {  // overflow split: the mains are the units of query blocks >= nxqb
        const int per = a.nqb - a.nxqb, um = (a.units / a.nqb) * per;
        const int mlo = x * um / 8, mn = (x + 1) * um / 8 - mlo;
        if (i < mn) unit = (mlo + i) / per * a.nqb + a.nxqb + (mlo + i) % per;
        return;
    }
    const int ulo = x * a.units / 8, un = (x + 1) * a.units / 8 - ulo;
    if (i < un) {
        unit = ulo + i;
        return;
    }
    int s = 0;
    for (int y = 0; y < x; ++y) s += (a.nprog - y + 7) / 8 - ((y + 1) * a.units / 8 - y * a.units / 8);
    spare = s + i - un;
}

template <int MODE>
__global__ __launch_bounds__(512) void attn_fwd_bf16_d128_split(const KArgs a) {
    constexpr int D = 128, BM = 256, BN = 32, NS = D / 16, NT = D / 32;
    constexpr int NB = 1;  // 32-row query blocks per wave (8 waves)
    constexpr int TILE = BN * D;  // elements of one K or V tile
    constexpr int NSTG = 5;       // LDS ring depth
    constexpr bool FAST = MODE == kDmaFast;
    // Tile t of a piece starting at tile tb lives in stage ((t - tb) mod 5): K
    // tiles in one region and V tiles in another, so every fragment read is a
    // per-lane base plus an immediate offset below 64 KB.
    __shared__ __attribute__((aligned(16))) uint16_t sK[NSTG * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t sV[NSTG * TILE];
    // Each wave's 32 query rows on their way in (Q) and out (bf16 O).
    __shared__ __attribute__((aligned(16))) uint16_t sQ[BM * D];
    __shared__ const uint16_t *sSegK[FAST ? 1 : kMaxKeyFrames];
    __shared__ const uint16_t *sSegV[FAST ? 1 : kMaxKeyFrames];
    __shared__ int sRedo;
    __shared__ int sPre[kMaxSplitUnits + 1];
    __shared__ int sTmp[256];
    lds_u16 *const kbase = (lds_u16 *)sK;
    lds_u16 *const vbase = (lds_u16 *)sV;

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, g = lane >> 5;

    if (!FAST) {
        for (int f = tid; f < a.nseg; f += 512) {
            sSegK[f] = (const uint16_t *)a.kseg[f];
            sSegV[f] = (const uint16_t *)a.vseg[f];
        }
    }
    build_piece_prefix(a, sPre, sTmp);  // ends with a barrier

    // Per-piece state.
    long hoff = 0;
    int qi[NB], lim[NB];
    bool qv[NB];
    bf16x8 qf[NB][NS];
    int nfull = 0, ntiles = 0;

    // DMA: this wave fills tile rows 4 wave + lr of K and of V, lane (lr, pch)
    // the physical 16-byte chunk pch, fetching the logical chunk that the
    // swizzle puts there.
    const int lr = lane >> 4, pch = lane & 15;
    lds_u16 *const qw = (lds_u16 *)sQ + wave * 32 * D;  // this wave's rows of sQ
    int qrow0 = 0;                                      // the piece's first row of this wave
    int kch[1], vch[1];
    uint32_t kvo[1], vvo[1];  // per-lane byte offsets from the group's first row
#pragma unroll
    for (int i = 0; i < 1; ++i) {
        kch[i] = pch ^ (4 * (wave & 3) + lr);           // (row mod 16) = 4 (wave mod 4) + lr
        vch[i] = (((pch >> 2) ^ lr) << 2) | (pch & 3);  // (row mod 4) = lr
        kvo[i] = (uint32_t)(((long)lr * a.ld + kch[i] * 8) * 2);
        vvo[i] = (uint32_t)(((long)lr * a.ld + vch[i] * 8) * 2);
    }
    const uint32_t k_lds = lds_addr(kbase), v_lds = lds_addr(vbase);
    auto m0k = [&](int S, int i) { return k_lds + (uint32_t)((S * TILE + (4 * wave + 4 * i) * D) * 2); };
    auto m0v = [&](int S, int i) { return v_lds + (uint32_t)((S * TILE + (4 * wave + 4 * i) * D) * 2); };

    // DMA cursor of this wave's 4-row group, as in the plain kernel: the
    // group's row drow inside segment dseg for the next tile to prefetch
    // (wave-uniform; a group never straddles two segments), turned by
    // prepare() into the tile's K and V addresses and moved one tile on, with
    // the segment's base pointers loaded one tile ahead, so that no
    // scalar-load wait sits at the barrier.  Past the last segment it wraps
    // inside the last one, so look-ahead tiles beyond the keys still read
    // valid (finite) rows, which the mask discards.  A segment is below 2^31
    // bytes.
    const int32_t ld2 = (int32_t)(a.ld * 2);
    int32_t hoff2 = 0;
    int drow = 0, dseg = 0;
    uint64_t dkp = 0, dvp = 0;
    SegPtrs nsp{};
    auto reset_cursor = [&](int tile) __attribute__((always_inline)) {
        const int j = tile * BN + 4 * wave;
        dseg = min(j / a.seg_len, a.nseg - 1);
        drow = j - dseg * a.seg_len;
        drow = drow >= a.seg_len ? drow - a.seg_len : drow;
        hoff2 = (int32_t)(hoff * 2);
        if constexpr (FAST) nsp = load_seg_ptrs_ahead(dseg);
    };
    auto prepare = [&]() __attribute__((always_inline)) {
        if constexpr (FAST) {
            const uint64_t off = (uint64_t)(uint32_t)(drow * ld2 + hoff2);
            dkp = nsp.k0 + off;
            dvp = nsp.v0 + off;
            drow += BN;
            const bool cr = drow >= a.seg_len;
            drow = cr ? drow - a.seg_len : drow;
            dseg = cr ? min(dseg + 1, a.nseg - 1) : dseg;
            nsp = load_seg_ptrs_ahead(dseg);
        }
    };
    auto issue = [&](int tile, auto S) {
        constexpr int st = decltype(S)::value;
        if constexpr (FAST) {
            dma16x2(dkp, dvp, kvo[0], vvo[0], m0k(st, 0), m0v(st, 0));
        } else {
            const int j0 = tile * BN;
#pragma unroll
            for (int i = 0; i < 1; ++i) {
                const int j = j0 + 4 * wave + 4 * i + lr;
                const uint16_t *kp = kZeroRow + kch[i] * 8;
                const uint16_t *vp = kZeroRow + vch[i] * 8;
                if (j < a.Tk) {
                    const int f = seg_of(j, a);
                    const long o = (long)(j - f * a.seg_len) * a.ld + hoff;
                    kp = sSegK[f] + o + kch[i] * 8;
                    vp = sSegV[f] + o + vch[i] * 8;
                }
                dma16_vaddr(kp, m0k(st, i));
                dma16_vaddr(vp, m0v(st, i));
            }
        }
    };

    // Per-lane LDS pointers of the fragment reads in stage 0; the stage, the
    // upper half of d and the key steps are immediate offsets.
    const lds_u16 *kfp[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) kfp[s] = kbase + n * D + (((2 * s + g) ^ (n & 15)) << 3);
    const int G = lane >> 4, sl = lane & 15;
    const int vrow = 4 * (G >> 1) + (sl >> 2);  // + 16 key-step + 8 half
    const lds_u16 *vfp[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        vfp[t] = vbase + vrow * D + ((2 * (t ^ (sl >> 2)) + (G & 1)) << 4) + 4 * (sl & 3);

    // Softmax with a fixed per-row exponent reference (log2 units): P =
    // exp2(s * c - mref).  mref is the row max of the row's first key tile, so
    // P <= 1 there; later tiles may exceed it, which is harmless while the
    // running sum stays far from the fp32 range.  A row whose sum ends above
    // 2^64 (or overflows) is recomputed in a second pass with its exact row max
    // as reference.  The accumulators are therefore touched only by MFMAs inside
    // the key loop.  Each row's result depends on its own scores only.  The row
    // sum adds the bf16-rounded P that the PV product uses.
    f32x16 acc[NB][NT];
    float mref[NB] = {0.f}, l[NB] = {0.f}, mmax[NB] = {-INFINITY};
    const float c = a.c;

    // Fragment reads of one tile: K (A operand of S^T = K Q^T, 8 k-steps over d)
    // and V^T (A operand of O^T += V^T P^T, 4 column blocks x 2 key steps, two
    // transposed 8-byte reads each).
    auto read_k = [&](auto S, bf16x8 *kf) {
        constexpr int st = decltype(S)::value;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            kf[s] = __builtin_bit_cast(bf16x8, *(lds_u32x4 *)(kfp[s] + st * TILE));
    };
    auto read_v = [&](auto S, v4i16 (*vf)[2][2]) {
        constexpr int st = decltype(S)::value;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                vf[t][s][0] = lds_tr16(vfp[t] + st * TILE + (16 * s) * D);
                vf[t][s][1] = lds_tr16(vfp[t] + st * TILE + (16 * s + 8) * D);
            }
    };
    // S^T = K Q^T: lane holds query n of each block and keys 8 (r/4) + 4 g + (r%4).
    auto qk = [&](const bf16x8 *kf, f32x16 *s) {
        s[0] = f32x16{};
#pragma unroll
        for (int st = 0; st < NS; ++st) s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[0][st], s[0], 0, 0, 0);
    };
    auto apply_mask = [&](f32x16 *s, int tile) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (tile * BN + 8 * (r >> 2) + 4 * g + (r & 3) >= lim[b]) s[b][r] = -INFINITY;
    };
    auto rowmax = [&](const f32x16 &s) {
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        return pair_max(mx);
    };
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    auto softmax = [&](const f32x16 *s, bf16x8 (*pf)[2], const float *mr) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pf[b][h][j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[b][8 * h + j], c, -mr[b]));
                const bf16x8 &p8 = pf[b][h];
                l[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 0, 1), ones, l[b], false);
                l[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 2, 3), ones, l[b], false);
                l[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 4, 5), ones, l[b], false);
                l[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 6, 7), ones, l[b], false);
            }
    };
    // O^T += V^T P^T.
    auto pv = [&](v4i16 (*vf)[2][2], bf16x8 (*pf)[2]) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const bf16x8 v = __builtin_bit_cast(
                    bf16x8, (v8i16)__builtin_shufflevector(vf[t][st][0], vf[t][st][1], 0, 1, 2, 3, 4, 5, 6, 7));
                acc[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, pf[0][st], acc[0][t], 0, 0, 0);
            }
    };

    // Software pipeline over key tiles, PV one tile behind the softmax.  Step
    // t (stage s(t) = t mod 5): wait until this wave's DMA of tile t+1 has
    // landed (t+2 may still be in flight), barrier (every wave's DMA of t+1 has
    // landed; every wave is done with step t-1, so the stage of tile t-2 is
    // free), then in one basic block: the K(t+1) fragment reads; O += V(t-1)
    // P(t-1) from registers, each MFMA followed by the transposed reads of the
    // V(t) fragments that take over its A operand's registers (they feed the
    // PV of step t+1); then S(t+1) = K(t+1) Q^T; the VALU turns S(t) into P(t)
    // under both; last the prefetch of tile t+3 into the stage of tile t-2.
    // The step after the last tile only adds the last PV (its tile is past
    // every row's limit, so its P is 0).
    //
    // Masked steps: a row whose limit lies at or below the tile start takes an
    // infinite exponent reference (P = 0); the element-wise mask runs only when
    // some row's limit falls inside the tile, at most a few tiles per block.
    // S and P in two register sets each, alternated by the unmasked steps as
    // in the plain kernel (PAR 2: the masked tail keeps set 0 and copies).
    f32x16 sbuf[2][NB];
    bf16x8 pbuf[2][NB][2];
    v4i16 vcur[NT][2][2];  // V^T fragments of the tile whose PV runs next
    auto step = [&](int t, auto S, auto masked, auto maxonly, auto par) __attribute__((always_inline)) {
        constexpr int s0 = decltype(S)::value;
        constexpr bool MASK = decltype(masked)::value;
        constexpr bool MAXONLY = decltype(maxonly)::value;
        constexpr int PAR = decltype(par)::value;
        constexpr bool COPY = PAR == 2;
        f32x16 stmp[NB];
        bf16x8 ptmp[NB][2];
        f32x16 *const scur = sbuf[COPY ? 0 : PAR];
        f32x16 *const snext = COPY ? stmp : sbuf[PAR ^ 1];
        bf16x8 (*const pprev)[2] = pbuf[COPY ? 0 : PAR];
        bf16x8 (*const pf)[2] = COPY ? ptmp : pbuf[PAR ^ 1];
        prepare();  // DMA addresses of tile t + 3
        // this wave's DMA of tile t+1 has landed (t+2 may still be in flight);
        // after the barrier every wave's has, and every wave is done with
        // step t-1, so the stage of tile t-2 is free
        __builtin_amdgcn_s_waitcnt(wait_vm(2));
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        float mr[NB] = {mref[0]};
        if (MASK) {
            const int t0 = t * BN;
            bool part = false;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                part = part || (lim[b] > t0 && lim[b] < t0 + BN);
                mr[b] = lim[b] <= t0 ? INFINITY : mref[b];
            }
            if (MAXONLY || __builtin_amdgcn_ballot_w64(part)) {
                asm volatile("");
                apply_mask(scur, t);
            }
        }
        bf16x8 kf[NS];
        read_k(std::integral_constant<int, (s0 + 1) % NSTG>{}, kf);
        __builtin_amdgcn_sched_barrier(0);  // the K reads go first
        if (MAXONLY) {
            qk(kf, snext);
#pragma unroll
            for (int b = 0; b < NB; ++b) mmax[b] = fmaxf(mmax[b], rowmax(scur[b]));
            issue(t + 3, std::integral_constant<int, (s0 + 3) % NSTG>{});
        } else {
            pv(vcur, pprev);
            read_v(std::integral_constant<int, s0>{}, vcur);
            softmax(scur, pf, mr);
            qk(kf, snext);
            issue(t + 3, std::integral_constant<int, (s0 + 3) % NSTG>{});
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
            if (COPY) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int h = 0; h < 2; ++h) pbuf[0][b][h] = ptmp[b][h];
            }
        }
        if (COPY) sbuf[0][0] = stmp[0];
    };
    auto sweep = [&](bool first_sweep, int tb, auto maxonly) __attribute__((always_inline)) {
        reset_cursor(tb);
        prepare();
        issue(tb, I0{});
        prepare();
        issue(tb + 1, I1{});
        prepare();
        issue(tb + 2, I2{});
        __builtin_amdgcn_s_waitcnt(wait_vm(4));  // tile 0 landed
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        if (first_sweep) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const bf16x8 v = lds_b128(qw + n * D + (((2 * s + g) ^ (n & 15)) << 3));
                qf[0][s] = qv[0] ? v : bf16x8{};
            }
        }
        {
            bf16x8 kf[NS];
            read_k(I0{}, kf);
            qk(kf, sbuf[0]);
        }
        if (first_sweep) {
            if (tb >= nfull) apply_mask(sbuf[0], tb);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float m = rowmax(sbuf[0][b]);
                mref[b] = m == -INFINITY ? 0.f : m * c;  // no key of the piece: P = 0 throughout
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h) pbuf[0][b][h] = bf16x8{};
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int ss = 0; ss < 2; ++ss) vcur[tt][ss][0] = vcur[tt][ss][1] = v4i16{0, 0, 0, 0};
        // Groups of five steps (static stages): unmasked while the whole group
        // is visible to every row, masked from there on, up to the step after
        // the last tile (which only adds the last PV).
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        using PC = std::integral_constant<int, 2>;
        int base = tb;
        if constexpr (FAST) {
#pragma unroll 1
            for (; base + 10 <= nfull; base += 10) {
                step(base, I0{}, std::false_type{}, maxonly, P0{});
                step(base + 1, I1{}, std::false_type{}, maxonly, P1{});
                step(base + 2, I2{}, std::false_type{}, maxonly, P0{});
                step(base + 3, I3{}, std::false_type{}, maxonly, P1{});
                step(base + 4, I4{}, std::false_type{}, maxonly, P0{});
                step(base + 5, I0{}, std::false_type{}, maxonly, P1{});
                step(base + 6, I1{}, std::false_type{}, maxonly, P0{});
                step(base + 7, I2{}, std::false_type{}, maxonly, P1{});
                step(base + 8, I3{}, std::false_type{}, maxonly, P0{});
                step(base + 9, I4{}, std::false_type{}, maxonly, P1{});
            }
        } else {
#pragma unroll 1
            for (; base + 5 <= nfull; base += 5) {
                step(base, I0{}, std::false_type{}, maxonly, PC{});
                step(base + 1, I1{}, std::false_type{}, maxonly, PC{});
                step(base + 2, I2{}, std::false_type{}, maxonly, PC{});
                step(base + 3, I3{}, std::false_type{}, maxonly, PC{});
                step(base + 4, I4{}, std::false_type{}, maxonly, PC{});
            }
        }
#pragma unroll 1
        for (; base <= ntiles; base += 5) {
            step(base, I0{}, std::true_type{}, maxonly, PC{});
            if (base + 1 > ntiles) break;
            step(base + 1, I1{}, std::true_type{}, maxonly, PC{});
            if (base + 2 > ntiles) break;
            step(base + 2, I2{}, std::true_type{}, maxonly, PC{});
            if (base + 3 > ntiles) break;
            step(base + 3, I3{}, std::true_type{}, maxonly, PC{});
            if (base + 4 > ntiles) break;
            step(base + 4, I4{}, std::true_type{}, maxonly, PC{});
        }
        // drain the look-ahead tiles before the stages are reused
        __builtin_amdgcn_s_waitcnt(wait_vm(0));
        compiler_fence();
    };

    // Tiles [tb, te) of unit (head, qb).  slot < 0: the whole unit, write O
    // (and LSE); else write the partial result (unnormalised O, reference,
    // sum) to workspace slot `slot`.
    auto do_piece = [&](int head, int qb, int tb, int te, int slot) __attribute__((always_inline)) {
        const int q0 = qb * BM;
        hoff = (long)head * D;
        const int lim_end = te * BN;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            qi[b] = q0 + 32 * NB * wave + 32 * b + n;
            qv[b] = qi[b] < a.Tq;
            lim[b] = min(key_limit(qv[b] ? qi[b] : a.Tq - 1, a), lim_end);
        }
        ntiles = te;
        nfull = min(te, min(key_limit(q0, a), lim_end) / BN);  // tiles visible to every row
        if (tid == 0) sRedo = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            l[b] = 0.f;
            mmax[b] = -INFINITY;
        }
        __syncthreads();
        // Q^T B operands: lane (n, g) holds q[qi][16 s + 8 g .. + 7]; the rows
        // go through the wave's part of sQ as in the plain kernel (DMA of whole
        // rows, fragments read back in the first sweep once tile 0 has landed).
        qrow0 = q0 + 32 * wave;
        if (qrow0 < a.Tq) {
            const uint64_t qp = (uint64_t)((const uint16_t *)a.q + (long)qrow0 * a.ld + hoff);
            const uint64_t qbase = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)qp) |
                                   ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(qp >> 32)) << 32);
            const int rmax = min(32, a.Tq - qrow0) - 1;
            // opaque copies: keeps the compiler from hoisting the eight lane
            // offsets out of the piece loop (they would be spilled)
            int lrp = lr, pchp = pch;
            asm volatile("" : "+v"(lrp), "+v"(pchp));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 4 * j + lrp;
                dma16(qbase, (uint32_t)(min(r, rmax) * ld2 + ((pchp ^ (r & 15)) << 4)),
                      lds_addr(qw) + (uint32_t)(j * 4 * D * 2));
            }
        }
    #pragma unroll
        for (int b = 0; b < NB; ++b)
    #pragma unroll
            for (int t = 0; t < NT; ++t) acc[b][t] = f32x16{};
        sweep(true, tb, std::false_type{});

        // Rare second pass for rows whose sum left the safe range.
        const float kSafeSum = 18446744073709551616.f;  // 2^64
        bool redo[NB];
    #pragma unroll
        for (int b = 0; b < NB; ++b) redo[b] = qv[b] && !(pair_sum(l[b]) <= kSafeSum);
        if (__builtin_amdgcn_ballot_w64(redo[0]) && lane == 0) sRedo = 1;
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(sRedo)) {
            asm volatile("");
            sweep(false, tb, std::true_type{});  // exact row maxima
            __syncthreads();
    #pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (redo[b]) mref[b] = mmax[b] * c;
                l[b] = 0.f;
    #pragma unroll
                for (int t = 0; t < NT; ++t) acc[b][t] = f32x16{};
            }
            sweep(false, tb, std::false_type{});
        }

    #pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float lt = pair_sum(l[b]);
            if (!qv[b]) continue;
            if (slot >= 0) {
                const int row = 32 * NB * wave + 32 * b + n;
                float *ps = a.ws + (long)slot * kSlotFloats;
    #pragma unroll
                for (int t = 0; t < NT; ++t)
    #pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *(f32x4 *)(ps + row * D + 32 * t + 8 * i + 4 * g) =
                            f32x4{acc[b][t][4 * i], acc[b][t][4 * i + 1], acc[b][t][4 * i + 2], acc[b][t][4 * i + 3]};
                if (g == 0) {
                    ps[BM * D + row] = mref[b];
                    ps[BM * D + BM + row] = lt;
                }
                continue;
            }
            const float inv = 1.f / lt;
            if (a.out_f32) {
                const long obase = (long)qi[b] * a.ld + hoff;
    #pragma unroll
                for (int t = 0; t < NT; ++t)
    #pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *(f32x4 *)((float *)a.o + obase + 32 * t + 8 * i + 4 * g) =
                            f32x4{acc[b][t][4 * i] * inv, acc[b][t][4 * i + 1] * inv,
                                  acc[b][t][4 * i + 2] * inv, acc[b][t][4 * i + 3] * inv};
            }
            if (g == 0 && a.lse) a.lse[(long)head * a.Tq + qi[b]] = mref[b] / kLog2e + logf(lt);
        }
        if (slot < 0 && !a.out_f32 && qrow0 < a.Tq) {
            // bf16 O of a whole unit through the wave's part of sQ, stored as
            // whole rows (as in the plain kernel)
            const float inv = 1.f / pair_sum(l[0]);
            int np = n, gp = g, lrp = lr, pchp = pch;  // opaque, as for the Q DMA
            asm volatile("" : "+v"(np), "+v"(gp), "+v"(lrp), "+v"(pchp));
    #pragma unroll
            for (int t = 0; t < NT; ++t)
    #pragma unroll
                for (int i = 0; i < 4; ++i)
                    *(__attribute__((address_space(3))) u32x2 *)(qw + np * D + (((4 * t + i) ^ (np & 15)) << 3) + 4 * gp) =
                        u32x2{pack_bf16x2(acc[0][t][4 * i] * inv, acc[0][t][4 * i + 1] * inv),
                              pack_bf16x2(acc[0][t][4 * i + 2] * inv, acc[0][t][4 * i + 3] * inv)};
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            compiler_fence();
    #pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 4 * j + lrp;
                const u32x4 v = *(lds_u32x4 *)(qw + r * D + (pchp << 3));
                if (qrow0 + r < a.Tq)
                    *(u32x4 *)((uint16_t *)a.o + (long)(qrow0 + r) * a.ld + hoff + ((pchp ^ (r & 15)) << 3)) = v;
            }
        }
        // Every wave is done with the stages and sRedo before the next piece.
        __syncthreads();

    };

    // Pieces of this workgroup: a main runs [0, min(n, T)) of its unit, a
    // spare its share of the tail pieces.
    int unit, spare;
    split_role(blockIdx.x, a, unit, spare);
    const bool ovf = a.nxqb > 0;
    auto run_tail = [&](int k) __attribute__((always_inline)) {
        const int pu = __builtin_amdgcn_readfirstlane(find_tail_unit(sPre, piece_units(a), k));
        const int i = k - __builtin_amdgcn_readfirstlane(sPre[pu]);
        const int u = piece_unit(pu, a);
        const int head = u / a.nqb, qb = u - head * a.nqb;
        const int tb = (ovf ? 0 : a.cut) + i * a.piece;
        const int te = min(block_tiles(qb, a), tb + a.piece);
        do_piece(head, qb, tb, te, (ovf ? 0 : a.units) + k);
    };
    if (unit >= 0) {
        const int head = unit / a.nqb, qb = unit - head * a.nqb;
        const int nt = block_tiles(qb, a);
        do_piece(head, qb, 0, min(nt, a.cut), nt > a.cut ? unit : -1);
        if (!ovf) return;
    }
    int k0, k1;
    if (ovf) {
        // every workgroup, after its main: XCD x takes pieces [x K / 8, (x +
        // 1) K / 8) (head-major, so mostly the heads of its own mains), shared
        // by its workgroups in order, lighter mains taking more (host plan)
        const int b = blockIdx.x;
        k0 = a.pk[b];
        k1 = b + 8 < a.nprog ? a.pk[b + 8] : (int)((long)((b & 7) + 1) * a.tail_total / 8);
    } else {
        k0 = (int)((long)spare * a.tail_total / a.nspare);
        k1 = (int)((long)(spare + 1) * a.tail_total / a.nspare);
    }
#pragma unroll 1
    for (int k = k0; k < k1; ++k) run_tail(k);
}

// Merges the pieces of every split unit of a split launch: with piece s holding
// acc_s (unnormalised O), reference m_s and sum l_s per row, M = max m_s over
// the pieces that saw keys, L = sum 2^(m_s - M) l_s, O = sum 2^(m_s - M) acc_s / L
// and LSE = M ln 2 + ln L.  Pieces are taken in a fixed order (main, then the
// tail pieces in order), so the result does not depend on timing.  Eight
// workgroups per unit, 32 rows each (thread: row tid / 8, 16 columns); units
// that were not split return at once.
constexpr int kCombineParts = 8;
__global__ __launch_bounds__(256) void attn_combine_d128(const KArgs a) {
    constexpr int D = 128, BM = kD128BM, RP = BM / kCombineParts;  // rows per workgroup
    const int tid = threadIdx.x;
    const int u = blockIdx.x / kCombineParts, part = blockIdx.x % kCombineParts;
    const int head = u / a.nqb, qb = u - head * a.nqb;
    const int q = unit_pieces(u, a);
    if (q == 0) return;
    int k0 = 0;  // tail pieces of the units before u (pieces depend on the query block only)
    for (int b = 0; b < a.nqb; ++b) {
        const int qb_pieces = unit_pieces(b, a);
        k0 += qb_pieces * head + (b < qb ? qb_pieces : 0);
    }
    // with an overflow split the unit has no main: its pieces are slots k0 ..
    const bool ovf = a.nxqb > 0;
    const int npieces = ovf ? q : 1 + q;
    auto slot_of = [&](int k) { return ovf ? k0 + k : (k == 0 ? u : a.units + k0 + k - 1); };
    const int row = part * RP + tid / 8, c0 = 16 * (tid % 8);
    const int qrow = qb * BM + row;

    // Both loops are unrolled and load every piece's statistics without a
    // branch (selecting afterwards), so that the loads of several pieces are
    // in flight together; the values and the order of the additions are those
    // of the plain loops.
    float M = -INFINITY;
#pragma unroll 4
    for (int k = 0; k < npieces; ++k) {
        const float *ps = a.ws + (long)slot_of(k) * kSlotFloats;
        const float ls = ps[BM * D + BM + row], ms = ps[BM * D + row];
        // ms is used either way (a piece without keys adds -inf, or NaN for
        // an infinite reference, which fmaxf drops), so its load is not
        // deferred behind the test of ls
        M = fmaxf(M, ms + (ls > 0.f ? 0.f : -INFINITY));
    }
    float L = 0.f;
    f32x4 o[4] = {};
#pragma unroll 4
    for (int k = 0; k < npieces; ++k) {
        const float *ps = a.ws + (long)slot_of(k) * kSlotFloats;
        const float ls = ps[BM * D + BM + row], ms = ps[BM * D + row];
        const float e = exp2f(ms - M);
        const float w = ls > 0.f ? e : 0.f;
        L += w * ls;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] += w * *(const f32x4 *)(ps + row * D + c0 + 4 * i);
    }
    if (qrow >= a.Tq) return;
    const float inv = 1.f / L;
    if (a.lse && tid % 8 == 0) a.lse[(long)head * a.Tq + qrow] = M / kLog2e + logf(L);
    const long off = (long)qrow * a.ld + (long)head * D + c0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 v = o[i] * inv;
        if (a.out_f32) {
            *(f32x4 *)((float *)a.o + off + 4 * i) = v;
        } else {
            const uint32_t b0 = __builtin_bit_cast(uint16_t, (__bf16)v[0]);
            const uint32_t b1 = __builtin_bit_cast(uint16_t, (__bf16)v[1]);
            const uint32_t b2 = __builtin_bit_cast(uint16_t, (__bf16)v[2]);
            const uint32_t b3 = __builtin_bit_cast(uint16_t, (__bf16)v[3]);
            *(u32x2 *)((uint16_t *)a.o + off + 4 * i) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
        }
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
    xcd_order(blockIdx.x, a.nwg, a.nqb, head, qb);
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

// Host mirror of block_tiles: key tiles of query block qb of the head_dim-128 kernel.
int64_t host_block_tiles(int64_t qb, const KArgs &k) {
    const int64_t last = std::min<int64_t>(qb * kD128BM + kD128BM - 1, k.Tq - 1);
    const int64_t lim = std::min<int64_t>((int64_t)k.prefix + (last / k.kpf + 1) * k.kpf, k.Tk);
    return (lim + kD128BN - 1) / kD128BN;
}

// Schedule of a split launch: the common cut T of the mains, tiles per tail
// piece, tail pieces in all and first-phase pieces per spare.
struct SplitPlan {
    int32_t cut, piece, pieces;
};

// Costs of the split schedule in units of one key-tile step of a main,
// measured on the Wan-1.3B step shape: a tail piece pays ~13 us beyond its
// tiles (Q load, pipeline fill, look-ahead drain, partial write), spares run
// their tiles ~1.35x slower than the mains (their K/V rows are rarely in L2),
// and merging a partial result costs ~0.01 step.  A split is taken only if it
// is predicted to be at least 10 % shorter than the plain launch.
constexpr double kPieceOverheadTiles = 16.0;
constexpr double kSpareTileCost = 1.35;
constexpr double kMergeTilesPerSlot = 0.01;
constexpr double kSplitMargin = 0.9;

// Chooses T, P and m by simulating the split schedule (see the work
// decomposition comment) on the problem's unit lengths; false when the split
// would not beat the plain launch by a margin.  Plans are cached per shape.
bool plan_split(const KArgs &k, int64_t H, int G, int64_t max_slots, double plain_steps, SplitPlan *out) {
    // Fixed-size storage throughout: planning allocates nothing (also on the
    // host), so callers that may not allocate can use the split path.
    struct Entry {
        int64_t key[7];
        bool ok;
        SplitPlan plan;
    };
    constexpr int kCache = 64;
    static std::mutex mu;
    static Entry cache[kCache];
    static int ncache = 0, next = 0;
    const int64_t key[7] = {k.Tq, k.Tk, k.kpf, k.prefix, H, G, max_slots};
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < ncache; ++i)
            if (std::equal(key, key + 7, cache[i].key)) {
                *out = cache[i].plan;
                return cache[i].ok;
            }
    }
    const int64_t nqb = k.nqb, U = nqb * H, S = G - U;
    if (nqb > kMaxSplitUnits || S <= 0) return false;
    int64_t nq[kMaxSplitUnits];
    int64_t nmax = 0, total = 0;
    for (int64_t qb = 0; qb < nqb; ++qb) {
        nq[qb] = host_block_tiles(qb, k);
        nmax = std::max(nmax, nq[qb]);
        total += nq[qb] * H;
    }
    const double ov = kPieceOverheadTiles;
    double best = plain_steps * kSplitMargin;  // the plain launch's makespan, less a margin
    bool ok = false;
    SplitPlan bp{};
    const int64_t kmax = std::min<int64_t>(max_slots - U, 2 * kMaxSplitUnits);
    int32_t len[2 * kMaxSplitUnits];
    const int64_t tlo = std::max<int64_t>(1, (int64_t)(0.7 * (double)total / (double)G));
    for (int32_t P : {8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256}) {
        for (int64_t T = tlo; T < nmax; ++T) {
            int64_t K = 0, split_units = 0;
            bool over = false;
            for (int64_t h = 0; h < H && !over; ++h)
                for (int64_t qb = 0; qb < nqb && !over; ++qb) {
                    const int64_t r = nq[qb] - T;
                    if (r > 0) ++split_units;
                    for (int64_t o = 0; o < r; o += P) {
                        if (K >= kmax) {
                            over = true;
                            break;
                        }
                        len[K++] = (int32_t)std::min<int64_t>(P, r - o);
                    }
                }
            if (over || K == 0) continue;
            double mk = (double)std::min(nmax, T) + ov;  // the mains
            for (int64_t s = 0; s < S; ++s) {             // the spares
                double f = 0.0;
                for (int64_t kk = s * K / S; kk < (s + 1) * K / S; ++kk) f += kSpareTileCost * len[kk] + ov;
                mk = std::max(mk, f);
            }
            mk += kMergeTilesPerSlot * (double)(split_units + K);
            if (mk < best) {
                best = mk;
                ok = true;
                bp = SplitPlan{(int32_t)T, P, (int32_t)K};
            }
        }
    }
    std::lock_guard<std::mutex> lock(mu);
    Entry &e = cache[next];
    next = (next + 1) % kCache;
    ncache = std::min(ncache + 1, kCache);
    std::copy(key, key + 7, e.key);
    e.ok = ok;
    e.plan = bp;
    *out = bp;
    return ok;
}

// Overflow split, for U units just beyond one round of G workgroups (U <=
// 1.5 G): the nx = ceil((U - G) / H) first query blocks of every head (the
// lightest under the frame mask) have no main; the others run whole on one
// workgroup each, and every workgroup then takes a contiguous run of the
// extra blocks' key tiles, cut into pieces of P tiles: each XCD's pieces go to
// its workgroups in order, as many as fit under a common finish time (found
// by bisection), so that workgroups with lighter mains take more.  The plain
// launch would run the extra blocks as a second round after the first compute
// units free up.  Costs as for plan_split; taken when predicted at least 10 %
// shorter.  Plans are kept per shape (fixed-size storage).
bool plan_overflow(const KArgs &k, int64_t H, int64_t G, int64_t max_slots, SplitPlan *out, int32_t *nxqb,
                   int16_t *pk) {
    struct Entry {
        int64_t key[7];
        bool ok;
        SplitPlan plan;
        int32_t nx;
        int16_t pk[kMaxSplitUnits];
    };
    constexpr int kCache = 16;
    static std::mutex mu;
    static Entry cache[kCache];
    static int ncache = 0, next = 0;
    const int64_t key[7] = {k.Tq, k.Tk, k.kpf, k.prefix, H, G, max_slots};
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < ncache; ++i)
            if (std::equal(key, key + 7, cache[i].key)) {
                *out = cache[i].plan;
                *nxqb = cache[i].nx;
                std::copy(cache[i].pk, cache[i].pk + kMaxSplitUnits, pk);
                return cache[i].ok;
            }
    }
    bool ok = false;
    SplitPlan bp{};
    int32_t bnx = 0;
    int16_t bpk[kMaxSplitUnits] = {};
    const int64_t nqb = k.nqb, U = nqb * H;
    const int64_t nx = (U - G + H - 1) / H;
    bool fit = U > G && 2 * U <= 3 * G && nx < nqb && nx * H <= kMaxSplitUnits && G <= kMaxSplitUnits;
    const int64_t um = U - nx * H, per = nqb - nx;
    for (int64_t x = 0; fit && x < 8; ++x)  // every XCD has a workgroup for each of its mains
        fit = (x + 1) * um / 8 - x * um / 8 <= (G - x + 7) / 8;
    if (fit) {
        int64_t nt[kMaxSplitUnits];
        int64_t nmax = 0, nmin_main = INT64_MAX, next_max = 0;
        for (int64_t qb = 0; qb < nqb && qb < kMaxSplitUnits; ++qb) {
            nt[qb] = host_block_tiles(qb, k);
            if (qb >= nx) {
                nmax = std::max(nmax, nt[qb]);
                nmin_main = std::min(nmin_main, nt[qb]);
            } else {
                next_max = std::max(next_max, nt[qb]);
            }
        }
        double mainlen[kMaxSplitUnits];  // per workgroup, as split_role assigns the mains
        for (int64_t b = 0; b < G; ++b) {
            const int64_t x = b & 7, i = b >> 3, mlo = x * um / 8, mn = (x + 1) * um / 8 - mlo;
            mainlen[b] = i < mn ? (double)nt[nx + (mlo + i) % per] + kPieceOverheadTiles : 0.0;
        }
        const double plain = (double)std::max(nmax, nmin_main + next_max);
        double best = plain * kSplitMargin;
        double cost[2 * kMaxSplitUnits];
        for (int32_t P : {8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512}) {
            int64_t K = 0;
            for (int64_t qb = 0; qb < nx; ++qb) K += H * ((nt[qb] + P - 1) / P);
            if (K > max_slots || K > 2 * kMaxSplitUnits) continue;
            {  // piece costs in piece order (head-major, then query block, then tiles)
                int64_t kk = 0;
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t qb = 0; qb < nx; ++qb)
                        for (int64_t t = 0; t < nt[qb]; t += P)
                            cost[kk++] = kSpareTileCost * (double)std::min<int64_t>(P, nt[qb] - t) + kPieceOverheadTiles;
            }
            double mk = 0.0;
            int16_t st[kMaxSplitUnits] = {};
            for (int64_t x = 0; x < 8; ++x) {
                const int64_t xlo = x * K / 8, xhi = (x + 1) * K / 8, nw = (G - x + 7) / 8;
                // fill the workgroups of XCD x in order up to finish time M;
                // returns the pieces left over
                auto fill = [&](double M, bool store) {
                    int64_t ptr = xlo;
                    for (int64_t i = 0; i < nw; ++i) {
                        const int64_t b = x + 8 * i;
                        if (store) st[b] = (int16_t)ptr;
                        double t = mainlen[b];
                        while (ptr < xhi && t + cost[ptr] <= M) t += cost[ptr++];
                    }
                    return xhi - ptr;
                };
                double lo = 0.0, hi = 0.0;
                for (int64_t i = 0; i < nw; ++i) lo = std::max(lo, mainlen[x + 8 * i]);
                hi = lo;
                for (int64_t kk = xlo; kk < xhi; ++kk) hi += cost[kk];
                for (int it = 0; it < 40; ++it) {
                    const double mid = 0.5 * (lo + hi);
                    if (fill(mid, false) == 0) hi = mid;
                    else lo = mid;
                }
                fill(hi, true);
                mk = std::max(mk, hi);
            }
            mk += kMergeTilesPerSlot * (double)K;
            if (mk < best) {
                best = mk;
                ok = true;
                bp = SplitPlan{1 << 30, P, (int32_t)K};
                bnx = (int32_t)nx;
                std::copy(st, st + kMaxSplitUnits, bpk);
            }
        }
    }
    std::lock_guard<std::mutex> lock(mu);
    Entry &e = cache[next];
    next = (next + 1) % kCache;
    ncache = std::min(ncache + 1, kCache);
    std::copy(key, key + 7, e.key);
    e.ok = ok;
    e.plan = bp;
    e.nx = bnx;
    std::copy(bpk, bpk + kMaxSplitUnits, e.pk);
    *out = bp;
    *nxqb = bnx;
    std::copy(bpk, bpk + kMaxSplitUnits, pk);
    return ok;
}

// Compute units of the current device, cached per device.
hipError_t cu_count(int *out) {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (const hipError_t e = hipGetDevice(&dev)) return e;
    if (dev >= 0 && dev < 64 && cache[dev].load() > 0) {
        *out = cache[dev].load();
        return hipSuccess;
    }
    int n = 0;
    if (const hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) return e;
    if (dev >= 0 && dev < 64) cache[dev].store(n);
    *out = n;
    return hipSuccess;
}

// Row mapping of the plain head_dim-128 launch (the GMAP of the kernel above;
// sets nqb, nwg and the mapping's KArgs).  Blocks of 256 consecutive rows,
// unless the launch fits in one round on the compute units and a paired
// mapping shortens the estimated longest block by 3 % or more.  Estimate: a
// block runs steps while any wave has tiles; a step costs 1 while some SIMD
// (waves w and w + 4) still has two working waves and 0.62 once every SIMD has
// at most one (as measured on the Wan-1.3B step): with a_s <= b_s the tiles of
// SIMD s's two groups, max a_s + 0.62 (max b_s - max a_s).  The frame-paired
// mapping needs groups aligned to frames that pad at most 1/64 of the rows.
struct RowPlan {
    int gm;
    int32_t nqb, nwr, wpf, nframes, w1;
    double steps;
};

RowPlan plan_rows_uncached(const KArgs &k, int64_t H, int cus);

// plan_rows with its results kept per problem shape (fixed-size storage, as
// for the split plans: planning allocates nothing).
int plan_rows(KArgs &k, int64_t H, int cus, double *steps) {
    struct Entry {
        int64_t key[6];
        RowPlan plan;
    };
    constexpr int kCache = 64;
    static std::mutex mu;
    static Entry cache[kCache];
    static int ncache = 0, next = 0;
    const int64_t key[6] = {k.Tq, k.Tk, k.kpf, k.prefix, H, cus};
    RowPlan rp{};
    bool hit = false;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < ncache && !hit; ++i)
            if (std::equal(key, key + 6, cache[i].key)) {
                rp = cache[i].plan;
                hit = true;
            }
    }
    if (!hit) {
        rp = plan_rows_uncached(k, H, cus);
        std::lock_guard<std::mutex> lock(mu);
        Entry &e = cache[next];
        next = (next + 1) % kCache;
        ncache = std::min(ncache + 1, kCache);
        std::copy(key, key + 6, e.key);
        e.plan = rp;
    }
    k.nqb = rp.nqb;
    k.nwg = (int)(rp.nqb * H);
    k.nwr = rp.nwr;
    k.wpf = rp.wpf;
    k.nframes = rp.nframes;
    k.w1 = rp.w1;
    *steps = rp.steps;
    return rp.gm;
}

RowPlan plan_rows_uncached(const KArgs &k, int64_t H, int cus) {
    const int64_t Tq = k.Tq, kpf = k.kpf;
    auto tiles_to = [&](int64_t row) {  // key tiles of the row's limit
        const int64_t lim = std::min<int64_t>(k.prefix + (row / kpf + 1) * kpf, k.Tk);
        return (lim + 31) / 32;
    };
    auto rows_tiles = [&](int64_t r0, int64_t nr) -> int64_t {
        return nr > 0 ? tiles_to(r0 + nr - 1) : 0;
    };
    // block cost from the tiles of its eight waves
    auto block_cost = [](const int64_t (&t)[8]) {
        int64_t ma = 0, mb = 0;
        for (int s = 0; s < 4; ++s) {
            ma = std::max(ma, std::min(t[s], t[s + 4]));
            mb = std::max(mb, std::max(t[s], t[s + 4]));
        }
        return (double)ma + 0.62 * (double)(mb - ma);
    };
    RowPlan rp{0, (int32_t)((Tq + 255) / 256), (int32_t)((Tq + 31) / 32), 0, 0, 0, 0.0};
    if ((int64_t)rp.nqb * H > cus) {
        // several rounds: the dispatcher balances them; the makespan estimate
        // is that of the heaviest block
        rp.steps = (double)tiles_to(Tq - 1);
        return rp;
    }
    double best = 0.0;
    for (int64_t b = 0; b < rp.nqb; ++b) {
        int64_t t[8];
        for (int w = 0; w < 8; ++w) {
            const int64_t r0 = 256 * b + 32 * w;
            t[w] = rows_tiles(r0, std::min<int64_t>(32, Tq - r0));
        }
        best = std::max(best, block_cost(t));
    }
    rp.steps = best;
    const double contiguous = best;
    // GMAP 1
    {
        const int64_t nwr = rp.nwr, nlight = (nwr + 1) / 2, nqb = (nlight + 3) / 4;
        double c = 0.0;
        for (int64_t b = 0; b < nqb; ++b) {
            int64_t t[8];
            for (int w = 0; w < 8; ++w) {
                const int64_t r = w < 4 ? 4 * b + w : nwr - 1 - (4 * b + w - 4);
                const bool ok = w < 4 ? r < nlight : r >= nlight;
                t[w] = ok ? rows_tiles(32 * r, std::min<int64_t>(32, Tq - 32 * r)) : 0;
            }
            c = std::max(c, block_cost(t));
        }
        if (nqb * H <= cus && c < best && c <= 0.97 * contiguous) {
            best = c;
            rp.gm = 1;
            rp.nqb = (int32_t)nqb;
            rp.steps = c;
        }
    }
    // GMAP 2
    const int64_t wpf = (kpf + 31) / 32, F = (Tq + kpf - 1) / kpf;
    if (F >= 2 && (wpf * 32 - kpf) * 64 <= kpf) {
        const int64_t np = F / 2, w1 = (wpf + 3) / 4, w2 = F % 2 ? (wpf + 7) / 8 : 0;
        const int64_t nqb = np * w1 + w2;
        auto group_tiles = [&](int64_t f, int64_t j) -> int64_t {
            if (j >= wpf) return 0;
            const int64_t r0 = f * kpf + 32 * j;
            return rows_tiles(r0, std::min(std::min<int64_t>(32, kpf - 32 * j), Tq - r0));
        };
        double c = 0.0;
        for (int64_t b = 0; b < nqb; ++b) {
            int64_t t[8];
            for (int w = 0; w < 8; ++w) {
                if (b < np * w1) {
                    const int64_t fp = b / w1, q = b - fp * w1;
                    t[w] = group_tiles(w < 4 ? fp : F - 1 - fp, 4 * q + (w & 3));
                } else {
                    t[w] = group_tiles(np, 8 * (b - np * w1) + w);
                }
            }
            c = std::max(c, block_cost(t));
        }
        if (nqb * H <= cus && c < best && c <= 0.97 * contiguous) {
            best = c;
            rp.gm = 2;
            rp.nqb = (int32_t)nqb;
            rp.wpf = (int32_t)wpf;
            rp.nframes = (int32_t)F;
            rp.w1 = (int32_t)w1;
            rp.steps = c;
        }
    }
    return rp;
}

template <int MODE>
void launch_plain(int gm, const KArgs &k, hipStream_t stream) {
    if (gm == 2)
        hipLaunchKernelGGL((attn_fwd_bf16_d128<MODE, 2>), dim3(k.nwg), dim3(512), 0, stream, k);
    else if (gm == 1)
        hipLaunchKernelGGL((attn_fwd_bf16_d128<MODE, 1>), dim3(k.nwg), dim3(512), 0, stream, k);
    else
        hipLaunchKernelGGL((attn_fwd_bf16_d128<MODE, 0>), dim3(k.nwg), dim3(512), 0, stream, k);
}

template <int D, bool SEG>
hipError_t launch_d(const KArgs &ka, const AttnProblem &p, hipStream_t stream) {
    KArgs k = ka;
    if (p.in_dtype == RTR_BF16 && D == 128) {
        k.nqb = (int)((p.Tq + 255) / 256);
        k.nwg = k.nqb * p.H;
        k.ws = nullptr;
        k.nprog = 0;
        int cu = 0;
        if (const hipError_t e = cu_count(&cu)) return e;
        // the plain launch's row mapping and estimated makespan
        KArgs kp = k;
        double plain_steps = 0.0;
        const int gm = plan_rows(kp, p.H, cu, &plain_steps);
        const int64_t U = (int64_t)k.nqb * p.H;
        const int64_t G = std::min<int64_t>(cu, kMaxSplitUnits);
        if (p.ws && U < G) {
            bool fit = true;  // every XCD has a workgroup for each of its mains
            for (int64_t x = 0; fit && x < 8; ++x) fit = (x + 1) * U / 8 - x * U / 8 <= (G - x + 7) / 8;
            SplitPlan plan{};
            const int64_t max_slots = p.ws_slots > 0 ? std::min<int64_t>(p.ws_slots, 2 * G) : 2 * G;
            if (fit && plan_split(k, p.H, (int)G, max_slots, plain_steps, &plan)) {
                k.ws = (float *)p.ws;
                k.nprog = (int32_t)G;
                k.units = (int32_t)U;
                k.cut = plan.cut;
                k.nspare = (int32_t)(G - U);
                k.tail_total = plan.pieces;
                k.piece = plan.piece;
            }
        } else if (p.ws && U > G) {
            const int64_t max_slots = p.ws_slots > 0 ? std::min<int64_t>(p.ws_slots, 2 * G) : 2 * G;
            SplitPlan plan{};
            int32_t nx = 0;
            if (plan_overflow(k, p.H, G, max_slots, &plan, &nx, k.pk)) {
                k.ws = (float *)p.ws;
                k.nprog = (int32_t)G;
                k.units = (int32_t)U;
                k.cut = plan.cut;
                k.nspare = 0;
                k.tail_total = plan.pieces;
                k.piece = plan.piece;
                k.nxqb = nx;
            }
        }
        const bool fast = k.seg_len >= 32 && k.seg_len % 4 == 0;
        if (k.nprog == 0) {
            if (fast)
                launch_plain<kDmaFast>(gm, kp, stream);
            else
                launch_plain<kDmaLane>(gm, kp, stream);
        } else {
            if (fast)
                hipLaunchKernelGGL((attn_fwd_bf16_d128_split<kDmaFast>), dim3(k.nprog), dim3(512), 0, stream, k);
            else
                hipLaunchKernelGGL((attn_fwd_bf16_d128_split<kDmaLane>), dim3(k.nprog), dim3(512), 0, stream, k);
            hipLaunchKernelGGL(attn_combine_d128, dim3(k.units * kCombineParts), dim3(256), 0, stream, k);
        }
    } else if (p.in_dtype == RTR_BF16) {
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

hipError_t attention_workspace_bytes(int32_t d, rtr_dtype in_dtype, size_t *bytes) {
    *bytes = 0;
    if (d != 128 || in_dtype != RTR_BF16) return hipSuccess;
    int cu = 0;
    if (const hipError_t e = cu_count(&cu)) return e;
    *bytes = (size_t)2 * std::min(cu, kMaxSplitUnits) * kSlotFloats * sizeof(float);
    return hipSuccess;
}

hipError_t plan_row_groups(int64_t Tq, int64_t Tk, int64_t kpf, int64_t prefix, int32_t H, RowGroups *out) {
    int cu = 0;
    if (const hipError_t e = cu_count(&cu)) return e;
    KArgs k{};
    k.Tq = (int32_t)Tq;
    k.Tk = (int32_t)Tk;
    k.kpf = (int32_t)kpf;
    k.prefix = (int32_t)prefix;
    double steps = 0.0;
    int gm = plan_rows(k, H, cu, &steps);
    if (gm != 2) {  // blocks of consecutive rows (GMAP 1 has no counterpart here)
        gm = 0;
        k.nqb = (int32_t)((Tq + 255) / 256);
    }
    out->gm = gm;
    out->nqb = k.nqb;
    out->wpf = k.wpf;
    out->nframes = k.nframes;
    out->w1 = k.w1;
    return hipSuccess;
}

hipError_t launch_attention(const AttnProblem &p, hipStream_t stream) {
    KArgs k{};
    k.q = p.q;
    k.o = p.o;
    k.lse = p.lse;
    for (int f = 0; f < p.nseg; ++f) {
        k.kseg[f] = p.kseg[f];
        k.vseg[f] = p.vseg[f];
    }
    k.kseg[p.nseg] = p.kseg[p.nseg - 1];
    k.vseg[p.nseg] = p.vseg[p.nseg - 1];
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
