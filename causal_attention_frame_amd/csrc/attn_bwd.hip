// Gradients of frame-block-causal attention for gfx950 (MI355X / CDNA4).
//
// dQ, dK, dV of Attn(Q,K,V) = softmax(Q K^T * scale + M) V, the equation of
// the RTR-DiT notes ("DiT as Real-Time Rerenderer ...", Key Designs 2), whose
// generator post-training (Key Designs 3) back-propagates through it.  From the
// forward's natural-log LSE, its output O and the upstream gradient dO, with
// P = exp(S - LSE) recomputed tile by tile and D_i = sum_c dO_ic O_ic:
//   dV = P^T dO,   dS = P * (dO V^T - D),   dK = scale dS^T Q,   dQ = scale dS K.
// The frame mask enters as in the forward: key j is seen by query i iff
// floor(j/k) <= floor(i/k), so a key is seen by every row from the first row
// of its own frame on, and a row by every key below the end of its frame.
//
// Kernels (head_dim 128, bf16 in and out, fp32 accumulation):
//   attn_bwd_prep       one 32-row tile per workgroup: -LSE / scale and -D
//                       per row, and the tile's Q and dO transposed into the
//                       layout the dK/dV kernel reads as MFMA A operands;
//   attn_bwd_dkdv_d128  one workgroup per 256 keys of a head, 8 waves of 32
//                       keys (two per SIMD): K stays in VGPRs as the MFMA B
//                       operand, V is staged once into LDS in the B operand's
//                       lane order, dK^T and dV^T (128 floats per lane) live in
//                       AGPRs, and the workgroup walks the 32-row query tiles
//                       that see its keys in a software pipeline (each MFMA
//                       phase beside independent VALU work), the tiles staged
//                       into LDS rings by DMA two tiles ahead;
//   attn_bwd_dq_d128    one workgroup per 256 query rows (8 waves x 32): Q and
//                       dO stay in registers, the workgroup walks the 32-key
//                       tiles its rows see in the same kind of software
//                       pipeline; dQ^T accumulates in registers.
// dQ is produced apart from dK/dV, recomputing S and dP, so that no partial
// sum leaves a workgroup: no atomics, and the result is deterministic.
//
// Streaming step (a chunk attending to the cached reference and window frames
// in front of it, Key Designs 4): the chunk rows see `prefix` cached keys and
// the chunk's own keys under the frame mask.  The prefix enters the chunk-key
// gradients only through LSE and D, so the chunk's dK/dV is the full form over
// the chunk; the prefix keys, seen by every row, are further dK/dV blocks of
// the same kernel that read their keys through a table of frame segments; and
// dQ walks the segment table over all keys.
//
// MFMA is v_mfma_f32_32x32x16_bf16.  Lane l of a wave is (n = l mod 32,
// g = l / 32).  An A operand lane holds row n and k = 8g..8g+7 of a 16-step;
// a B operand lane column n and the same k; accumulator element r of a lane is
// row 8 (r/4) + 4 g + (r mod 4), column n.  A 32x32 accumulator can therefore
// serve directly as the B operand of a product that contracts over its rows:
// k-step h takes elements 8h..8h+7, i.e. rows 16h + 8 (e/4) + 4g + (e mod 4)
// for e = 0..7, and the A operand reads its k positions in that same order.

#include <algorithm>
#include <climits>
#include <cmath>
#include <type_traits>

#include "device_util.h"
#include "rtr_internal.h"

namespace rtr {
namespace {

using namespace dev;

struct BArgs {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;
    uint16_t *dq, *dk, *dv;
    // [H][nqt][64]: -LSE / scale of the tile's 32 rows, then their -D.  The
    // dK/dV kernel loads them as the initial values of the S and dP
    // accumulators, which then hold S - LSE / scale (P = exp2(c S)) and dP - D.
    float *rows;
    uint16_t *qt;  // [H][nqt][4096]: transposed Q tiles
    uint16_t *dot; // [H][nqt][4096]: transposed dO tiles
    int32_t T, kpf, nqt;
    int32_t nkb, nqb;  // 256-key blocks, 256-row blocks per head
    int32_t nwg;       // workgroups of the current launch
    int64_t ld;        // row stride in elements (H * 128)
    float c;           // scale * log2(e)
    float scale;
    // Streaming step: keys [0, Tk) lie in segments of seg_len keys (row
    // j - f seg_len of the [*, H, 128] block at kseg[f] / vseg[f]); the first
    // `prefix` are seen by every query row.  The full form has Tk = T and no
    // prefix.  dkp/dvp receive the prefix keys' gradients ([prefix][H][128]);
    // nkbp counts their 256-key blocks per head (0: not wanted).
    const void *kseg[kMaxKeyFrames], *vseg[kMaxKeyFrames];
    int32_t nseg, seg_len;
    float inv_seg_len;
    int32_t prefix, Tk, nkbp;
    uint16_t *dkp, *dvp;
    // Prefix-key blocks split over the query tiles (few keys, many rows: the
    // text of a cross-attention): piece p of a block walks tiles
    // [p tpp, (p + 1) tpp) and leaves unscaled fp32 dK^T / dV^T partials in
    // part[p][key][head][2][128], summed in piece order by attn_bwd_reduce.
    int32_t nsplit, tpp;
    float *part;
    // Row groups of the dQ launch (its GMAP instance; RowGroups): groups per
    // frame, frames, and workgroups per frame pair.
    int32_t wpf, nframes, w1;
};

constexpr int kD = 128;
constexpr int kTile = 32 * kD;  // elements of one 32-row tile

// Position p (0..31) of a transposed tile row holds query row swap23(p) of the
// tile: within each 16-row step the middle two groups of four trade places, so
// that an A operand lane's eight k positions 8g..8g+7 of step h are the rows
// 16h + 8 (e/4) + 4g + (e mod 4) that the accumulator layout assigns to it.
__device__ inline int swap23(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// Transposed tile: row d (0..127) of 32 positions = four 16-byte chunks; chunk
// c of row d is stored at chunk c ^ ((d / 4) mod 4), so that the 16 lanes of
// one LDS pass (rows d..d+15, one logical chunk) touch 16 distinct bank groups.

// Row-major 32x128 tile staged for plain reads only: chunk c (8 columns) of
// row r at chunk c ^ (r mod 16).
__device__ inline int swz_plain(int r) { return r & 15; }
// Row-major tile read both plainly (16-byte reads of 16 rows) and transposed
// (ds_read_b64_tr_b16: one pass serves 32 lanes, 4 rows x 64 bytes): chunk c
// of row r at chunk c ^ s(r), s(r) = 4 (r mod 4) + (r / 4 mod 4) -- a
// permutation of 0..15 over any 16 consecutive rows, whose values shifted
// right by two also differ over any 4 consecutive rows starting at a multiple
// of 4, so neither read has a bank conflict.
__device__ inline int swz_dual(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Segment holding key j (the float estimate corrected by one step).
__device__ inline int seg_of(int j, const BArgs &a) {
    int f = (int)((float)j * a.inv_seg_len);
    const int rem = j - f * a.seg_len;
    if (rem < 0) --f;
    else if (rem >= a.seg_len) ++f;
    return f;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; the clobber is still honoured
// DMA of 16 bytes per lane from a per-lane 64-bit address to LDS byte address
// m0 + 16 * lane (rows from a segment table have no common base).
__device__ inline void dma16_lane(const void *src, uint32_t m0a) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(m0a)
                 : "memory", "m0");
}
// The DMA form of dma16 (device_util.h) issued by lanes 0 and 1 only: exec is
// narrowed and restored inside the statement, so that the caller's code stays
// one basic block (a branch there lets the compiler sink VALU work across the
// barrier that follows).
__device__ inline void dma16_lanes01(uint64_t b0, uint32_t o0, uint32_t m0a) {
    uint64_t saved;
    asm volatile(
        "s_mov_b64 %0, exec\n\ts_mov_b64 exec, 3\n\ts_mov_b32 m0, %2\n\ts_nop 4\n\t"
        "global_load_lds_dwordx4 %1, %3\n\ts_mov_b64 exec, %0"
        : "=&s"(saved)
        : "v"(o0), "s"(m0a), "s"(b0)
        : "memory", "m0");
}
#pragma clang diagnostic pop

// mfma_acc (device_util.h) without its wait states, for operands that no
// VALU instruction wrote within the last few instructions (LDS loads, or
// values formed a whole phase earlier).
__device__ inline void mfma_acc_ready(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Row statistics and transposed tiles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_bwd_prep(const BArgs a) {
    __shared__ uint16_t sT[2][kD][33];  // [Q, dO][d][row], padded against bank conflicts
    const int tile = blockIdx.x, head = blockIdx.y;
    const int tid = threadIdx.x, r = tid >> 3, c8 = tid & 7;  // row, 16-column group
    const int qrow = tile * 32 + r;
    const bool valid = qrow < a.T;
    const long off = (long)qrow * a.ld + (long)head * kD + 16 * c8;
    u32x4 qv[2] = {}, dv[2] = {}, ov[2] = {};
    if (valid) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            qv[h] = gload16(a.q + off + 8 * h);
            dv[h] = gload16(a.dout + off + 8 * h);
            ov[h] = gload16(a.o + off + 8 * h);
        }
    }
    float dsum = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            dsum = fmaf(bf_lo(dv[h][w]), bf_lo(ov[h][w]), dsum);
            dsum = fmaf(bf_hi(dv[h][w]), bf_hi(ov[h][w]), dsum);
        }
    dsum += __shfl_xor(dsum, 1);
    dsum += __shfl_xor(dsum, 2);
    dsum += __shfl_xor(dsum, 4);
    float *rows = a.rows + ((long)head * a.nqt + tile) * 64;
    if (c8 == 0) {
        rows[r] = valid ? -a.lse[(long)head * a.T + qrow] / a.scale : -INFINITY;
        rows[32 + r] = valid ? -dsum : 0.f;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int d = 16 * c8 + 8 * h + 2 * w;
            sT[0][d][r] = (uint16_t)qv[h][w];
            sT[0][d + 1][r] = (uint16_t)(qv[h][w] >> 16);
            sT[1][d][r] = (uint16_t)dv[h][w];
            sT[1][d + 1][r] = (uint16_t)(dv[h][w] >> 16);
        }
    __syncthreads();
    const long tbase = ((long)head * a.nqt + tile) * kTile;
#pragma unroll
    for (int zz = 0; zz < 2; ++zz) {
        const int z = tid + 256 * zz;  // output chunk: row d, stored chunk pc
        const int d = z >> 2, pc = z & 3, lc = pc ^ ((d >> 2) & 3);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int p = 8 * lc + 2 * e;
                w[e] = (uint32_t)sT[t][d][swap23(p)] | ((uint32_t)sT[t][d][swap23(p + 1)] << 16);
            }
            *(u32x4 *)((t ? a.dot : a.qt) + tbase + 8 * z) = w;
        }
    }
}

// ---------------------------------------------------------------------------
// dK and dV: one workgroup per 256 keys, 8 waves of 32 keys.
// ---------------------------------------------------------------------------
// One LDS array: a 3-stage ring of query tiles' row-major and transposed Q
// (16 KB per stage), a 2-stage ring of their row-major and transposed dO and
// row statistics (16.25 KB per stage), then the workgroup's V rows (64 KB):
// step s of wave w at RV + (8 w + s) 512 + 8 lane, one lane-linear 16-byte read.
constexpr int kDkdvLds = 10 * kTile + 2 * 128 + 256 * kD;  // uint16 units

// Key block kb of a head: the query rows' own keys (PRE false: the full form,
// or the chunk's keys of a streaming step) or the cached prefix keys (PRE
// true), which every query row sees and which are read through the segment
// table.  lbase: LDS byte address of the kDkdvLds array.
template <bool PRE>
__device__ __attribute__((always_inline)) inline void dkdv_block(const BArgs &a, int head, int kb, int piece,
                                                                 uint32_t lbase) {
    constexpr int NS = 8, NT = 4;
    constexpr int RQ = 0, RQT = 3 * kTile, RDO = 6 * kTile, RDOT = 8 * kTile;  // in uint16 units
    constexpr int RROW = 10 * kTile;
    constexpr int RV = RROW + 2 * 128;
    const bool pre = PRE;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7, two per SIMD
    const int n = lane & 31, g = lane >> 5;
    const int k0 = kb * 256;
    const long hoff = (long)head * kD;

    // This lane's key (column n of the wave's S tiles) and the first row that sees it.
    const int kj = k0 + 32 * wave + n;
    const int nkeys = pre ? a.prefix : a.T;
    const bool kvalid = kj < nkeys;
    const int qmin = pre ? 0 : (kj / a.kpf) * a.kpf;
    const int t0 = pre ? piece * a.tpp : ((k0 / a.kpf) * a.kpf) / 32;  // first tile that sees a key of the block
    const int nt = pre ? min(a.tpp, a.nqt - t0) : a.nqt - t0;
    // Tiles that start below the first row of the block's last key frame may
    // hold rows that miss some of its keys: they take the element-wise mask.
    const int last_key = min(k0 + 255, a.T - 1);
    const int nmask = pre ? 0 : min(nt, max(0, ((last_key / a.kpf) * a.kpf - t0 * 32 + 31) / 32));

    // K as B operands in registers (lane (n, g): row kj, columns 16 s + 8 g ..),
    // V rows of the same lanes DMA'd into LDS.
    bf16x8 kf[NS];
    if constexpr (PRE) {
        const int jj = kvalid ? kj : a.prefix - 1;
        const int f = seg_of(jj, a);
        const long o = (long)(jj - f * a.seg_len) * a.ld + hoff + 8 * g;
        const uint16_t *kr = (const uint16_t *)a.kseg[f] + o, *vr = (const uint16_t *)a.vseg[f] + o;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            kf[s] = __builtin_bit_cast(bf16x8, gload16(kr + 16 * s));
            dma16_lane(vr + 16 * s, lbase + 2 * (RV + (wave * NS + s) * 512));
        }
    } else {
        const long ro = (long)(kvalid ? kj : a.T - 1) * a.ld + hoff;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            kf[s] = __builtin_bit_cast(bf16x8, gload16(a.k + ro + 16 * s + 8 * g));
            dma16((uint64_t)a.v, (uint32_t)((ro + 16 * s + 8 * g) * 2), lbase + 2 * (RV + (wave * NS + s) * 512));
        }
    }
    // Complete these loads here: otherwise the compiler's wait for them sits
    // inside the tile loop, where it would also drain the DMA ring.
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    compiler_fence();
    const uint32_t pv = lbase + 2 * (RV + wave * NS * 512 + 8 * lane);

    // DMA of query tile i into Q stage qs and dO stage ds, 5 loads per wave:
    // row-major Q and dO (wave w fills rows 4w + lr, lane (lr, pch) the stored
    // chunk pch), the two transposed tiles (contiguous 8 KB, wave w its 1 KB)
    // and the row statistics (32 bytes per wave, lanes 0 and 1).
    const int lr = lane >> 4, pch = lane & 15;
    const int prow = 4 * wave + lr;
    const uint32_t plain_col = (uint32_t)(16 * (pch ^ swz_plain(prow)));
    const uint32_t l0 = lbase + 1024 * wave;
    auto issue = [&](int i, int qs, int ds) __attribute__((always_inline)) {
        const int tq = min(t0 + i, a.nqt - 1);
        const int row = min(tq * 32 + prow, a.T - 1);
        const uint32_t off = (uint32_t)(((long)row * a.ld + hoff) * 2) + plain_col;
        dma16x2((uint64_t)a.q, (uint64_t)a.dout, off, off, l0 + 2 * (RQ + qs * kTile), l0 + 2 * (RDO + ds * kTile));
        const long tb = ((long)head * a.nqt + tq) * kTile * 2 + 1024 * wave;
        dma16x2((uint64_t)a.qt + tb, (uint64_t)a.dot + tb, 16u * lane, 16u * lane, l0 + 2 * (RQT + qs * kTile),
                l0 + 2 * (RDOT + ds * kTile));
        const uint64_t rb = (uint64_t)(a.rows + ((long)head * a.nqt + tq) * 64 + 8 * wave);
        dma16_lanes01(rb, 16u * lane, lbase + 2 * (RROW + ds * 128) + 32 * wave);
    };

    // Fragment addresses (bytes; a stage's offset is added per step, the
    // region's is an immediate).  Plain read of k-step s (row n, logical chunk
    // 2s + g, stored at (2s + g) ^ (n mod 16)) at aq ^ 32 s.  Transposed read
    // of row d = 32 t + n, k-step h (logical chunk 2h + g, stored at
    // (2h + g) ^ (n/4 mod 4)) at pt[h] + 2048 t.  Row statistics of rows
    // 8 j + 4 g .. + 3: -LSE / scale at pr + 32 j, -D 128 bytes further.
    uint32_t pt[2];
    const uint32_t aq = lbase + 2 * (n * kD + 8 * (g ^ swz_plain(n)));
#pragma unroll
    for (int h = 0; h < 2; ++h) pt[h] = lbase + 2 * (n * 32 + 8 * ((2 * h + g) ^ ((n >> 2) & 3)));
    const uint32_t pr = lbase + 2 * RROW + 16 * g;
    auto rd = [](uint32_t addr, int imm) __attribute__((always_inline)) {
        return lds_b128((const lds_u16 *)(uintptr_t)addr + imm / 2);
    };
    auto rd4 = [](uint32_t addr, int imm) __attribute__((always_inline)) {
        return *(const lds_f32x4 *)((const lds_u16 *)(uintptr_t)addr + imm / 2);
    };

    f32x16 dkt[NT], dvt[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) dkt[t] = dvt[t] = f32x16{};
    const float c = a.c;

    // The walk over the query tiles is software-pipelined so that the MFMAs
    // of each phase have independent VALU or LDS work beside them (the two
    // waves of a SIMD otherwise run the same phase at the same time, and the
    // matrix core idles through both waves' softmax).  Iteration i, with
    // s = S(i) - LSE / scale already computed (S = Q K^T; the accumulator
    // starts at -LSE / scale, so P = exp2(c s)):
    //   1. dP - D = dO(i) V^T - D; the VALU turns s into P;
    //   2. dV^T += dO(i)^T P; the VALU forms dS = P (dP - D);
    //   wait for this wave's DMA of tile i+1, barrier (every wave's has
    //   landed; every wave is done with tile i's dO and with tile i-1's Q),
    //   DMA of tile i+2 into those stages;
    //   3. dK^T += Q(i)^T dS and s = S(i+1) - LSE / scale.
    // Q thus takes three stages (phase 3 reads tiles i and i+1), dO two.  The
    // last iteration's S(i+1) reads a clamped tile and is discarded.
    f32x16 s;
    // s = -LSE / scale of the rows whose statistics lie at bst: the start of
    // their S accumulation.
    auto s_init = [&](uint32_t bst) __attribute__((always_inline)) {
        f32x4 i4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) i4[j] = rd4(bst, 32 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[4 * j + e] = i4[j][e];
    };

    // Phase 1's first loads, issued at the end of the previous phase 3: the
    // -D rows of the tile (the dP accumulator's start) and its first two
    // fragment pairs.
    struct Ahead {
        f32x4 i4[4];
        bf16x8 fa[2], fb[2];
    } ah;
    // Part p (0..3) of those loads for the tile in dO stage ds.
    auto load_ahead = [&](int p, int ds) __attribute__((always_inline)) {
        if (p < 2) {
#pragma unroll
            for (int j = 2 * p; j < 2 * p + 2; ++j) ah.i4[j] = rd4(pr + (uint32_t)(ds * 256), 128 + 32 * j);
        } else {
            ah.fa[p - 2] = rd((aq + (uint32_t)(ds * kTile * 2)) ^ (32u * (p - 2)), 2 * RDO);
            ah.fb[p - 2] = rd(pv, 1024 * (p - 2));
        }
    };

    auto iter = [&](int i, int qs, int qn, int ds, auto masked) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(masked)::value;
        const uint32_t sod = (uint32_t)(ds * kTile * 2), soq = (uint32_t)(qs * kTile * 2);
        const uint32_t bdo = aq + sod;
        // dO^T at btd + 2 (RDOT - RDO) + 2048 t (the region's full offset would
        // not fit the 16-bit immediate), Q^T at btq + 2 RQT + 2048 t.
        const uint32_t btd[2] = {pt[0] + 2 * RDO + sod, pt[1] + 2 * RDO + sod};
        const uint32_t btq[2] = {pt[0] + soq, pt[1] + soq};

        // Phase 1: dP - D = dO V^T - D (the accumulator starts at -D) under
        // P = exp2(c s), one element pair per MFMA.
        f32x16 dp;
        bf16x8 pb[2];
        {
            bf16x8 fa[NS], fb[NS];
            uint32_t pw[2][4];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                fa[k] = ah.fa[k];
                fb[k] = ah.fb[k];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) dp[4 * j + e] = ah.i4[j][e];
            fa[2] = rd(bdo ^ (32u * 2), 2 * RDO);
            fb[2] = rd(pv, 1024 * 2);
            __builtin_amdgcn_sched_barrier(0);
            const int q0 = (t0 + i) * 32 + 4 * g;
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k], fb[k], dp, 0, 0, 0);
                if (k + 3 < NS) {
                    fa[k + 3] = rd(bdo ^ (32u * (k + 3)), 2 * RDO);
                    fb[k + 3] = rd(pv, 1024 * (k + 3));
                }
                const int r = 2 * k, row = q0 + 8 * (r >> 2) + (r & 3);
                float p0 = __builtin_amdgcn_exp2f(s[r] * c), p1 = __builtin_amdgcn_exp2f(s[r + 1] * c);
                if (MASK) {
                    p0 = row >= qmin ? p0 : 0.f;
                    p1 = row + 1 >= qmin ? p1 : 0.f;
                }
                s[r] = p0;
                s[r + 1] = p1;
                pw[k >> 2][k & 3] = pack_bf16x2(p0, p1);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) pb[h] = __builtin_bit_cast(bf16x8, u32x4{pw[h][0], pw[h][1], pw[h][2], pw[h][3]});
        }

        // Phase 2: dV^T += dO^T P under dS = P (dP - D), one element pair per
        // MFMA; the first dK^T fragments are read at its end.
        bf16x8 sb[2], fk[NS];
        {
            bf16x8 fv[NS];
            uint32_t sw[2][4];
#pragma unroll
            for (int k = 0; k < 4; ++k) fv[k] = rd(btd[k & 1], 2 * (RDOT - RDO) + 2048 * (k >> 1));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                if (k < 2) mfma_acc(dvt[k >> 1], fv[k], pb[k & 1]);
                else mfma_acc_ready(dvt[k >> 1], fv[k], pb[k & 1]);
                if (k + 4 < NS) fv[k + 4] = rd(btd[k & 1], 2 * (RDOT - RDO) + 2048 * ((k + 4) >> 1));
                else fk[k - 4] = rd(btq[k & 1], 2 * RQT + 2048 * ((k - 4) >> 1));
                const int r = 2 * k;
                sw[k >> 2][k & 3] = pack_bf16x2(s[r] * dp[r], s[r + 1] * dp[r + 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) sb[h] = __builtin_bit_cast(bf16x8, u32x4{sw[h][0], sw[h][1], sw[h][2], sw[h][3]});
        }

        __builtin_amdgcn_s_waitcnt(wait_vm(0));  // this wave's loads of tile i+1 landed
        lds_barrier();                            // everyone's have; tile i's dO and tile i-1's Q are free
        issue(i + 2, qn == 2 ? 0 : qn + 1, ds);

        // Phase 3: dK^T += Q^T dS and S(i+1) = Q(i+1) K^T - LSE / scale,
        // alternating, each fragment read two MFMA pairs ahead.
        {
            const uint32_t bq = aq + (uint32_t)(qn * kTile * 2);
            bf16x8 fq[NS];
            s_init(pr + (uint32_t)((ds ^ 1) * 256));
#pragma unroll
            for (int k = 0; k < 3; ++k) fq[k] = rd(bq ^ (32u * k), 2 * RQ);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                mfma_acc_ready(dkt[k >> 1], fk[k], sb[k & 1]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[k], kf[k], s, 0, 0, 0);
                if (k + 4 < NS) fk[k + 4] = rd(btq[k & 1], 2 * RQT + 2048 * ((k + 4) >> 1));
                if (k + 3 < NS) fq[k + 3] = rd(bq ^ (32u * (k + 3)), 2 * RQ);
                if (k >= 4) load_ahead(k - 4, ds ^ 1);  // tile i+1
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    if (nt > 0) {
        issue(0, 0, 0);
        issue(1, 1, 1);
        __builtin_amdgcn_s_waitcnt(wait_vm(0));
        lds_barrier();
        s_init(pr);  // S(0)
#pragma unroll
        for (int k = 0; k < NS; ++k) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd(aq ^ (32u * k), 2 * RQ), kf[k], s, 0, 0, 0);
#pragma unroll
        for (int p = 0; p < 4; ++p) load_ahead(p, 0);
    }
    int i = 0, qs = 0, ds = 0;
#pragma unroll 1
    for (; i < nmask; ++i) {
        const int qn = qs == 2 ? 0 : qs + 1;
        iter(i, qs, qn, ds, std::true_type{});
        qs = qn;
        ds ^= 1;
    }
#pragma unroll 1
    for (; i < nt; ++i) {
        const int qn = qs == 2 ? 0 : qs + 1;
        iter(i, qs, qn, ds, std::false_type{});
        qs = qn;
        ds ^= 1;
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // no DMA outlives the workgroup's LDS
    acc_settle();  // before the AGPR reads below

    if (!kvalid) return;
    if (PRE && a.nsplit > 1) {  // one piece of a split block: fp32 partials, reduced later
        float *const pp = a.part + ((long)piece * a.prefix + kj) * (2 * a.ld) + 2 * hoff;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 32 * t + 8 * j + 4 * g;
                const f32x16 &k_ = dkt[t], &v_ = dvt[t];
                *(f32x4 *)(pp + d0) = f32x4{k_[4 * j], k_[4 * j + 1], k_[4 * j + 2], k_[4 * j + 3]};
                *(f32x4 *)(pp + kD + d0) = f32x4{v_[4 * j], v_[4 * j + 1], v_[4 * j + 2], v_[4 * j + 3]};
            }
        return;
    }
    const long ob = (long)kj * a.ld + hoff;
    uint16_t *const dko = pre ? a.dkp : a.dk, *const dvo = pre ? a.dvp : a.dv;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d0 = 32 * t + 8 * j + 4 * g;
            const f32x16 &k_ = dkt[t], &v_ = dvt[t];
            *(u32x2 *)(dko + ob + d0) = u32x2{pack_bf16x2(k_[4 * j] * a.scale, k_[4 * j + 1] * a.scale),
                                               pack_bf16x2(k_[4 * j + 2] * a.scale, k_[4 * j + 3] * a.scale)};
            *(u32x2 *)(dvo + ob + d0) = u32x2{pack_bf16x2(v_[4 * j], v_[4 * j + 1]),
                                               pack_bf16x2(v_[4 * j + 2], v_[4 * j + 3])};
        }
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_d128(const BArgs a) {
    __shared__ __attribute__((aligned(256))) uint16_t smem[kDkdvLds];
    __shared__ int sMap[2];
    int head, blk;
    xcd_order_shared(blockIdx.x, a.nwg, a.nkb + a.nkbp * a.nsplit, head, blk, sMap);
    // Blocks of cached prefix keys (streaming step; every row sees them, so
    // they carry the most work) take the highest indices, then the blocks of
    // the query rows' own keys, earliest keys highest.
    const uint32_t lbase = lds_addr((lds_u16 *)smem);
    if (blk >= a.nkb)
        dkdv_block<true>(a, head, (blk - a.nkb) / a.nsplit, (blk - a.nkb) % a.nsplit, lbase);
    else
        dkdv_block<false>(a, head, a.nkb - 1 - blk, 0, lbase);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 256 query rows.  SEG: keys through the segment table
// (streaming step), otherwise one contiguous [T, H, 128] block.  GMAP 0: wave
// w of block qb takes rows 256 qb + 32 w .. + 31; GMAP 2 (one-round launches
// with several frames): 32-row groups aligned to frames, frame f paired with
// frame F-1-f, so that each SIMD (waves w and w + 4) holds an early and a late
// group (RowGroups).  A wave whose rows all lie before a key tile skips its
// products from there on (it still loads its share of the tiles and meets the
// barriers).
// ---------------------------------------------------------------------------
template <bool SEG, int GMAP>
__global__ __launch_bounds__(512) void attn_bwd_dq_d128(const BArgs a) {
    constexpr int NS = 8, NT = 4, NSTG = 4;
    __shared__ __attribute__((aligned(16))) uint16_t sK[NSTG * kTile];
    __shared__ __attribute__((aligned(16))) uint16_t sV[NSTG * kTile];
    __shared__ const uint16_t *sSegK[SEG ? kMaxKeyFrames : 1], *sSegV[SEG ? kMaxKeyFrames : 1];

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, g = lane >> 5;

    __shared__ int sMap[2];
    int head, qb;
    xcd_order_shared(blockIdx.x, a.nwg, a.nqb, head, qb, sMap);
    const long hoff = (long)head * kD;
    auto key_limit = [&](int i) __attribute__((always_inline)) {
        return (int)min((long)a.prefix + (long)(i / a.kpf + 1) * a.kpf, (long)a.Tk);
    };
    // first row and row count (0: none) of wave w's group
    auto wave_rows = [&](int w, int &r0, int &nr) __attribute__((always_inline)) {
        r0 = 0;
        nr = 0;
        if constexpr (GMAP == 0) {
            r0 = 256 * qb + 32 * w;
            nr = min(32, a.T - r0);
        } else {
            // blocks counted from the last one, as in the forward kernel
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
                nr = min(min(32, a.kpf - 32 * j), a.T - r0);
            }
        }
        nr = max(nr, 0);
    };
    int r0w, nrw;
    wave_rows(wave, r0w, nrw);
    const int qi = r0w + n;
    const bool qv = n < nrw;
    // Key limits grow with the row: a wave's largest is its last row's, the
    // block's the largest over its waves.
    const int lim_wave = nrw > 0 ? key_limit(r0w + nrw - 1) : 0;
    int lim_blk = 0;
#pragma unroll 1
    for (int w = 0; w < 8; ++w) {
        int r0, nr;
        wave_rows(w, r0, nr);
        if (nr > 0) lim_blk = max(lim_blk, key_limit(r0 + nr - 1));
    }
    if (SEG) {
        for (int f = tid; f < a.nseg; f += 512) {
            sSegK[f] = (const uint16_t *)a.kseg[f];
            sSegV[f] = (const uint16_t *)a.vseg[f];
        }
        __syncthreads();
    }
    const int lim = key_limit(qv ? qi : a.T - 1);
    const int ntiles = (lim_blk + 31) / 32;
    // tiles every row of this wave sees whole (none for a wave without rows)
    const int nfull = nrw > 0 ? min(ntiles, key_limit(r0w) / 32) : 0;

    // Q and dO as B operands: lane (n, g) holds row qi, columns 16 s + 8 g .. + 7.
    bf16x8 qf[NS], df[NS];
    {
        const long ro = (long)(qv ? qi : a.T - 1) * a.ld + hoff;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qf[s] = __builtin_bit_cast(bf16x8, gload16(a.q + ro + 16 * s + 8 * g));
            df[s] = __builtin_bit_cast(bf16x8, gload16(a.dout + ro + 16 * s + 8 * g));
        }
    }
    float l2 = INFINITY, dd = 0.f;
    if (qv) {
        const float *rs = a.rows + ((long)head * a.nqt + qi / 32) * 64;
        l2 = -rs[qi & 31] * a.c;  // LSE in log2 units
        dd = -rs[32 + (qi & 31)];
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // as in the dK/dV kernel: no load wait inside the loop
    compiler_fence();

    // DMA of one key tile: K and V rows 4w + lr, lane (lr, pch) the stored chunk pch.
    const int lr = lane >> 4, pch = lane & 15;
    const int prow = 4 * wave + lr;
    const uint32_t col2 = (uint32_t)(16 * (pch ^ swz_dual(prow)));
    const uint32_t lk = lds_addr((lds_u16 *)sK), lv = lds_addr((lds_u16 *)sV);
    auto issue = [&](int j, auto S) __attribute__((always_inline)) {
        constexpr int st = decltype(S)::value;
        const int row = min(j * 32 + prow, a.Tk - 1);
        if (SEG) {
            const int f = seg_of(row, a);
            const long o = (long)(row - f * a.seg_len) * a.ld + hoff + col2 / 2;
            dma16_lane(sSegK[f] + o, lk + st * kTile * 2 + 1024 * wave);
            dma16_lane(sSegV[f] + o, lv + st * kTile * 2 + 1024 * wave);
        } else {
            const uint32_t off = (uint32_t)(((long)row * a.ld + hoff) * 2) + col2;
            dma16x2((uint64_t)a.k, (uint64_t)a.v, off, off, lk + st * kTile * 2 + 1024 * wave,
                    lv + st * kTile * 2 + 1024 * wave);
        }
    };

    // Plain reads (A operand of S^T = K Q^T and dP^T = V dO^T: key row n,
    // k = 16 s + 8 g ..).
    const lds_u16 *pk[NS], *pv[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int o = n * kD + 8 * ((2 * s + g) ^ swz_dual(n));
        pk[s] = (lds_u16 *)sK + o;
        pv[s] = (lds_u16 *)sV + o;
    }
    // Transposed reads (A operand of dQ^T = K^T dS^T: row d = 32 t + n, k-step h
    // at keys 16 h + 4 g + 0..3 and 16 h + 8 + 4 g + 0..3).  ds_read_b64_tr_b16:
    // the 16 lanes of group G read a 4-row x 16-column block, lane sl giving the
    // address of row sl/4, columns 4 (sl mod 4) .. + 3, and receive column sl.
    const int G = lane >> 4, sl = lane & 15;
    const lds_u16 *ptr[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int r = 4 * (G >> 1) + (sl >> 2) + 8 * e;
            const int ch = 4 * t + 2 * (G & 1) + ((sl & 3) >> 1);
            ptr[t][e] = (lds_u16 *)sK + r * kD + 8 * (ch ^ swz_dual(r)) + 4 * (sl & 1);
        }

    f32x16 dqt[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) dqt[t] = f32x16{};
    const float c = a.c;

    // The walk over the key tiles is software-pipelined as in the dK/dV
    // kernel.  Iteration j (stage j mod 4), with s = S^T(j) = K(j) Q^T:
    //   1. dP^T = V(j) dO^T; the VALU turns s into P = exp2(s c - LSE2);
    //   wait for this wave's DMA of tile j+1, barrier (every wave's has
    //   landed; every wave is done with tile j-1), DMA of tile j+3 into the
    //   stage of tile j-1;
    //   2. S^T(j+1) = K(j+1) Q^T; the VALU forms dS = P (dP - D);
    //   3. dQ^T += K(j)^T dS^T.
    // One element pair of the VALU work per MFMA, each fragment read two
    // MFMAs ahead.  The last iteration's S^T(j+1) reads a clamped tile and is
    // discarded.
    f32x16 s;
    auto iter = [&](int j, auto S, auto masked) __attribute__((always_inline)) {
        constexpr int st = decltype(S)::value, st1 = (st + 1) % NSTG;
        constexpr bool MASK = decltype(masked)::value;
        if (MASK && j * 32 >= lim_wave) {
            // tile j and later lie past every row of this wave (P = 0): only
            // the loads and the barrier (masked loop only, so that the
            // unmasked iterations stay one basic block)
            __builtin_amdgcn_s_waitcnt(wait_vm(2));
            lds_barrier();
            issue(j + 3, std::integral_constant<int, (st + 3) % NSTG>{});
            return;
        }

        // Phase 1: dP^T = V dO^T under P = exp2(s c - LSE2).
        f32x16 dp = {};
        {
            bf16x8 fa[NS];
#pragma unroll
            for (int k = 0; k < 2; ++k) fa[k] = lds_b128(pv[k] + st * kTile);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k], df[k], dp, 0, 0, 0);
                if (k + 2 < NS) fa[k + 2] = lds_b128(pv[k + 2] + st * kTile);
                const int r = 2 * k, key = j * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                float p0 = __builtin_amdgcn_exp2f(fmaf(s[r], c, -l2)), p1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], c, -l2));
                if (MASK) {
                    p0 = key < lim ? p0 : 0.f;
                    p1 = key + 1 < lim ? p1 : 0.f;
                }
                s[r] = p0;
                s[r + 1] = p1;
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        __builtin_amdgcn_s_waitcnt(wait_vm(2));  // this wave's loads of tile j+1 landed
        lds_barrier();                            // everyone's have; tile j-1 is free
        issue(j + 3, std::integral_constant<int, (st + 3) % NSTG>{});

        // Phase 2: S^T(j+1) = K(j+1) Q^T under dS = P (dP - D).
        f32x16 sn = {};
        bf16x8 sb[2];
        {
            bf16x8 fa[NS];
            uint32_t sw[2][4];
#pragma unroll
            for (int k = 0; k < 2; ++k) fa[k] = lds_b128(pk[k] + st1 * kTile);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k], qf[k], sn, 0, 0, 0);
                if (k + 2 < NS) fa[k + 2] = lds_b128(pk[k + 2] + st1 * kTile);
                const int r = 2 * k;
                sw[k >> 2][k & 3] = pack_bf16x2(s[r] * (dp[r] - dd), s[r + 1] * (dp[r + 1] - dd));
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) sb[h] = __builtin_bit_cast(bf16x8, u32x4{sw[h][0], sw[h][1], sw[h][2], sw[h][3]});
        }

        // Phase 3: dQ^T += K^T dS^T (fragment k: d block k/2, k-step k mod 2).
        {
            bf16x8 kt[NS];
            auto rd_kt = [&](int k) __attribute__((always_inline)) {
                return cat_tr(lds_tr16(ptr[k >> 1][0] + st * kTile + 16 * (k & 1) * kD),
                              lds_tr16(ptr[k >> 1][1] + st * kTile + 16 * (k & 1) * kD));
            };
#pragma unroll
            for (int k = 0; k < 2; ++k) kt[k] = rd_kt(k);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                dqt[k >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[k], sb[k & 1], dqt[k >> 1], 0, 0, 0);
                if (k + 2 < NS) kt[k + 2] = rd_kt(k + 2);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        s = sn;
        // In the masked loop, whose iterations are separated by exit tests,
        // S^T(j+1) is formed here rather than sunk past an exit.
        if (MASK) asm volatile("" : "+v"(s));
    };

    issue(0, I0{});
    issue(1, I1{});
    issue(2, I2{});
    __builtin_amdgcn_s_waitcnt(wait_vm(4));  // tile 0 landed
    lds_barrier();
    {
        s = f32x16{};
#pragma unroll
        for (int k2 = 0; k2 < NS; k2 += 4) {
            bf16x8 fa[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) fa[k] = lds_b128(pk[k2 + k]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 4; ++k) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k], qf[k2 + k], s, 0, 0, 0);
        }
    }
    int j = 0;
#pragma unroll 1
    for (; j + 4 <= nfull; j += 4) {
        iter(j, I0{}, std::false_type{});
        iter(j + 1, I1{}, std::false_type{});
        iter(j + 2, I2{}, std::false_type{});
        iter(j + 3, I3{}, std::false_type{});
    }
#pragma unroll 1
    for (; j < ntiles; j += 4) {
        iter(j, I0{}, std::true_type{});
        if (j + 1 >= ntiles) break;
        iter(j + 1, I1{}, std::true_type{});
        if (j + 2 >= ntiles) break;
        iter(j + 2, I2{}, std::true_type{});
        if (j + 3 >= ntiles) break;
        iter(j + 3, I3{}, std::true_type{});
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    compiler_fence();

    if (!qv) return;
    const long ob = (long)qi * a.ld + hoff;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * t + 8 * i + 4 * g;
            *(u32x2 *)(a.dq + ob + d0) = u32x2{pack_bf16x2(dqt[t][4 * i] * a.scale, dqt[t][4 * i + 1] * a.scale),
                                               pack_bf16x2(dqt[t][4 * i + 2] * a.scale, dqt[t][4 * i + 3] * a.scale)};
        }
}

// Sum of the pieces of split prefix-key blocks, in piece order: four
// consecutive floats of one (key, head) row per thread; dK scaled, both to bf16.
__global__ __launch_bounds__(256) void attn_bwd_reduce(const BArgs a) {
    const long e = (long)blockIdx.x * 256 + threadIdx.x;  // f32x4 index
    const long per_piece = (long)a.prefix * 2 * a.ld;     // floats per piece
    if (e * 4 >= per_piece) return;
    f32x4 acc = {};
    for (int p = 0; p < a.nsplit; ++p) acc += *(const f32x4 *)(a.part + p * per_piece + e * 4);
    const long row = e / 64;           // (key, head) row of 256 floats
    const int c = (int)(e % 64) * 4;   // 0..255: dK columns, then dV columns
    const long key = row / (a.ld / kD), head = row % (a.ld / kD);
    const bool isk = c < kD;
    const float f = isk ? a.scale : 1.f;
    uint16_t *const dst = (isk ? a.dkp : a.dvp) + key * a.ld + head * kD + (c & (kD - 1));
    *(u32x2 *)dst = u32x2{pack_bf16x2(acc[0] * f, acc[1] * f), pack_bf16x2(acc[2] * f, acc[3] * f)};
}

// Pieces per prefix-key block: split only when the blocks alone would leave
// most of the GPU idle, into pieces of at least 16 query tiles.
int bwd_split(int64_t T, int32_t H, int64_t prefix, bool cross) {
    const int64_t nqt = (T + 31) / 32, wg = (int64_t)H * ((prefix + 255) / 256);
    if (!cross || wg >= 128 || nqt < 32) return 1;
    const int64_t want = std::min<int64_t>((256 + wg - 1) / wg, nqt / 16);
    const int64_t tpp = (nqt + want - 1) / want;
    return (int)((nqt + tpp - 1) / tpp);
}

}  // namespace

hipError_t attention_cross_bwd_workspace_bytes(int64_t Tq, int64_t n, int32_t H, size_t *bytes) {
    if (const hipError_t e = attention_bwd_workspace_bytes(Tq, H, bytes)) return e;
    const int ns = bwd_split(Tq, H, n, true);
    if (ns > 1) *bytes = (*bytes + 255) / 256 * 256 + (size_t)ns * n * H * 2 * kD * sizeof(float);
    return hipSuccess;
}

hipError_t attention_bwd_workspace_bytes(int64_t T, int32_t H, size_t *bytes) {
    const int64_t nqt = (T + 31) / 32;
    *bytes = (size_t)(H * nqt) * (64 * sizeof(float) + 2 * kTile * sizeof(uint16_t));
    return hipSuccess;
}

hipError_t launch_attention_bwd(const BwdProblem &p, hipStream_t stream) {
    if (p.T == 0) return hipSuccess;
    BArgs a{};
    a.q = (const uint16_t *)p.q;
    a.k = (const uint16_t *)p.k;
    a.v = (const uint16_t *)p.v;
    a.o = (const uint16_t *)p.o;
    a.dout = (const uint16_t *)p.dout;
    a.lse = p.lse;
    a.dq = (uint16_t *)p.dq;
    a.dk = (uint16_t *)p.dk;
    a.dv = (uint16_t *)p.dv;
    a.T = (int32_t)p.T;
    a.kpf = (int32_t)std::min<int64_t>(p.tokens_per_frame, p.T);
    a.nqt = (int32_t)((p.T + 31) / 32);
    a.nqb = (int32_t)((p.T + 255) / 256);
    a.nkb = p.cross ? 0 : a.nqb;  // blocks of the rows' own keys (none for cross-attention)
    a.ld = (int64_t)p.H * kD;
    a.scale = p.scale;
    a.c = p.scale * kLog2e;
    const int64_t ntile = (int64_t)p.H * a.nqt;
    a.rows = (float *)p.ws;
    a.qt = (uint16_t *)(a.rows + ntile * 64);
    a.dot = a.qt + ntile * kTile;
    a.Tk = a.T;
    a.seg_len = a.T;
    // A streaming step with an empty prefix is the full form over the chunk.
    const bool seg = p.nseg > 0 && p.prefix > 0;
    if (seg) {
        for (int f = 0; f < p.nseg; ++f) {
            a.kseg[f] = p.kseg[f];
            a.vseg[f] = p.vseg[f];
        }
        a.nseg = p.nseg;
        a.seg_len = (int32_t)p.seg_len;
        a.prefix = (int32_t)p.prefix;
        a.Tk = a.prefix + (p.cross ? 0 : a.T);
        if (p.dk_prefix) {
            a.nkbp = (int32_t)((p.prefix + 255) / 256);
            a.dkp = (uint16_t *)p.dk_prefix;
            a.dvp = (uint16_t *)p.dv_prefix;
            a.nsplit = bwd_split(p.T, p.H, p.prefix, p.cross);
            a.tpp = (a.nqt + a.nsplit - 1) / a.nsplit;
            if (a.nsplit > 1) {
                size_t prep = 0;
                if (const hipError_t e = attention_bwd_workspace_bytes(p.T, p.H, &prep)) return e;
                a.part = (float *)((char *)p.ws + (prep + 255) / 256 * 256);
            }
        }
    }
    a.inv_seg_len = 1.0f / (float)a.seg_len;
    if (a.nsplit == 0) {
        a.nsplit = 1;
        a.tpp = a.nqt;
    }

    hipLaunchKernelGGL(attn_bwd_prep, dim3(a.nqt, p.H), dim3(256), 0, stream, a);
    if (hipError_t e = hipGetLastError()) return e;
    a.nwg = p.H * (a.nkb + a.nkbp * a.nsplit);
    if (a.nwg > 0) {  // none: cross-attention whose text is not differentiated
        hipLaunchKernelGGL(attn_bwd_dkdv_d128, dim3(a.nwg), dim3(512), 0, stream, a);
        if (hipError_t e = hipGetLastError()) return e;
    }
    if (a.nsplit > 1) {
        const long n4 = (long)a.prefix * 2 * a.ld / 4;
        hipLaunchKernelGGL(attn_bwd_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, a);
        if (hipError_t e = hipGetLastError()) return e;
    }
    // dQ: the row mapping of the forward launch over the same rows and keys
    RowGroups rg{};
    if (const hipError_t e = plan_row_groups(a.T, a.Tk, a.kpf, a.prefix, p.H, &rg)) return e;
    a.nqb = rg.nqb;
    a.wpf = rg.wpf;
    a.nframes = rg.nframes;
    a.w1 = rg.w1;
    a.nwg = p.H * a.nqb;
    if (rg.gm == 2) {
        if (seg)
            hipLaunchKernelGGL((attn_bwd_dq_d128<true, 2>), dim3(a.nwg), dim3(512), 0, stream, a);
        else
            hipLaunchKernelGGL((attn_bwd_dq_d128<false, 2>), dim3(a.nwg), dim3(512), 0, stream, a);
    } else {
        if (seg)
            hipLaunchKernelGGL((attn_bwd_dq_d128<true, 0>), dim3(a.nwg), dim3(512), 0, stream, a);
        else
            hipLaunchKernelGGL((attn_bwd_dq_d128<false, 0>), dim3(a.nwg), dim3(512), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace rtr
