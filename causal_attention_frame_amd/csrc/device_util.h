// Device-side helpers shared by the gfx950 attention kernels: vector types,
// the XCD-aware work order, LDS access and global-to-LDS DMA.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace rtr {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(1))) const u32x4 global_u32x4;

constexpr float kLog2e = 1.4426950408889634f;

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2,
// and an XCD starts its workgroups in index order as compute units free up.
// Every XCD gets one contiguous head-major range of work items, so the blocks
// of one head (which read the same tensors) share an L2, and runs that range
// by block index, highest first, across its heads.  Callers number blocks so
// that the highest index carries the most work.  Within a head, work item
// position p holds block perm(p), alternating between the heaviest and the
// lightest remaining blocks (nblk-1, 0, nblk-2, 1, ...): an XCD whose range
// cuts a head in two then gets about its share of that head's work, where
// ranges of consecutive blocks gave one XCD the heavy half and its neighbour
// the light half.
//
// With lo = A nblk + a and hi - 1 = B nblk + bl, the heads whose position p
// lies in the range are A + [p < a] .. B - [p > bl], so the walk over the
// blocks needs two divisions in all (integer divisions by a variable are long
// instruction sequences; one per block and head bound cost the last
// workgroups of a 20-block launch ~3 us before their first key tile).
__host__ __device__ inline void xcd_order(int b, int nwg, int nblk, int &head, int &blk) {
    const int x = b & 7, i = b >> 3;
    const int q8 = nwg >> 3, r8 = nwg & 7;
    const int lo = x * q8 + (x < r8 ? x : r8), hi = lo + q8 + (x < r8 ? 1 : 0);
    const int half = nblk >> 1;
    const int A = lo / nblk, a = lo - A * nblk;
    const int B = (hi - 1) / nblk, bl = (hi - 1) - B * nblk;
    int rem = i;
    head = A;
    blk = a;  // not reached for a valid b
    for (int q = nblk - 1; q >= 0; --q) {
        const int p = q >= half ? 2 * (nblk - 1 - q) : 2 * q + 1;  // position of block q
        const int hmin = A + (p < a ? 1 : 0), hmax = B - (p > bl ? 1 : 0);
        const int cnt = hmax - hmin + 1;
        if (cnt <= 0) continue;
        if (rem < cnt) {
            head = hmin + rem;
            blk = q;
            return;
        }
        rem -= cnt;
    }
}

// xcd_order for the whole workgroup, walked by its first wave and shared
// through smap (two ints of LDS): the waves of a compute unit share one scalar
// unit, so every wave walking the blocks itself took eight times as long (up
// to ~3 us before the first key tile of a 20-block launch).  Ends with a
// workgroup barrier.
__device__ inline void xcd_order_shared(int b, int nwg, int nblk, int &head, int &blk, int *smap) {
    if (threadIdx.x < 64) {
        int h, q;
        xcd_order(b, nwg, nblk, h, q);
        if (threadIdx.x == 0) {
            smap[0] = h;
            smap[1] = q;
        }
    }
    __syncthreads();
    head = __builtin_amdgcn_readfirstlane(smap[0]);
    blk = __builtin_amdgcn_readfirstlane(smap[1]);
}

__device__ inline uint32_t lds_addr(const lds_u16 *p) { return (uint32_t)(uintptr_t)p; }

__device__ inline v4i16 lds_tr16(const lds_u16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p);
}

__device__ inline bf16x8 lds_b128(const lds_u16 *p) { return __builtin_bit_cast(bf16x8, *(lds_u32x4 *)p); }

__device__ inline bf16x8 cat_tr(v4i16 lo, v4i16 hi) {
    return __builtin_bit_cast(bf16x8, (v8i16)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ inline u32x4 gload16(const uint16_t *p) { return *(const global_u32x4 *)p; }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; the clobber is still honoured
// Two DMA loads, each 16 bytes per lane from global memory to LDS byte address
// m0 + 16 * lane; source: a wave-uniform 64-bit base in SGPRs plus a per-lane
// 32-bit byte offset.  The s_nop 4 covers the wait states after an m0 write
// and after a VALU write of an SGPR that a vector memory instruction reads
// (every SGPR operand is written before the statement, so one guard covers
// both loads); the second m0 write needs one.
__device__ inline void dma16x2(uint64_t b0, uint64_t b1, uint32_t o0, uint32_t o1, uint32_t m0a, uint32_t m0b) {
    asm volatile(
        "s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %4\n\t"
        "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %5"
        :
        : "v"(o0), "v"(o1), "s"(m0a), "s"(m0b), "s"(b0), "s"(b1)
        : "memory", "m0");
}
// One DMA load of the same form.
__device__ inline void dma16(uint64_t b0, uint32_t o0, uint32_t m0a) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %2"
                 :
                 : "v"(o0), "s"(m0a), "s"(b0)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// acc += A B with the accumulator held in AGPRs.  Files that use it are built
// with builtin MFMAs in VGPR form (their results feed VALU code), and their
// long-lived accumulators live in AGPRs through this statement instead, which
// leaves the VGPRs to the rest of the kernel.  The s_nop covers a VALU write of
// an A or B operand just before; the hardware forwards an exactly matching
// accumulator from the previous MFMA of the same shape.  Before other code
// touches the accumulator registers, acc_settle() waits out the last MFMA.
__device__ inline void mfma_acc(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last accumulating MFMA and other reads or writes
// of its AGPRs (more than the 18 a 16-pass MFMA needs).
__device__ inline void acc_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
constexpr int wait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)

__device__ inline void compiler_fence() { asm volatile("" ::: "memory"); }

// Barrier after this wave's LDS reads have completed.
__device__ inline void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// Two floats to a bf16 pair (round to nearest even), lo in the low half.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)lo, (__bf16)hi});
}

}  // namespace dev
}  // namespace rtr
