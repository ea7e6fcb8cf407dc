// lds_pipe.h -- gfx950 helpers for staging tiles into LDS without registers
// and reading MFMA operands out of them.
//
//  * dma16() / dma4(): global_load_lds_dwordx4 / _dword -- each lane copies
//    16 (4) bytes from (wave-uniform global base) + (its 32-bit offset) into
//    LDS at (wave-uniform LDS base) + 16 (4) * lane.  The copies count in
//    vmcnt like loads; they are waited for with an explicit s_waitcnt
//    vmcnt(n) and made visible to the workgroup with s_barrier.  They are
//    issued from asm (no register results; the "memory" clobber keeps LDS
//    accesses on their side of the issue): the compiler then never waits
//    for them on its own -- it cannot tell every LDS read from a copy in
//    flight and would otherwise drain all copies before such reads -- and
//    the waits written here are the only ones that order them.  Each sets
//    M0 (the copy's LDS base) inside its own asm; hipcc warns that M0 is a
//    reserved register in the clobber list.  The kernels' compiled code
//    reads M0 nowhere else: every M0 access in their ISA is one of these
//    s_mov_b32 m0 writes directly before its copy.
//  * tr16(): ds_read_b64_tr_b16 -- within each group of 16 lanes, lane i
//    receives element (i % 4) of the 4-element (8-byte) rows addressed by
//    lanes 4k + i/4, k = 0..3.  If lane r of a group addresses row (token)
//    t0 + r/4 at column quad q(r % 4), lane i gets 4 consecutive tokens of
//    column q(i/4) + i%4: the K-contiguous operand fragment of a token-major
//    tile.
//  * Row swizzles: the 16-byte chunk index inside an LDS row is XORed with a
//    function of the row so that the operand reads hit distinct banks.  The
//    copy side realises the swizzle by choosing, for LDS slot c', the global
//    chunk c = c' ^ f(row).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

#define SSD_LDS __attribute__((address_space(3)))

namespace ssd {

typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_addr(const SSD_LDS void* p) {
    return (uint32_t)(uintptr_t)p;
}
// base: wave-uniform global address; voff: per-lane byte offset; ldst:
// wave-uniform LDS address of lane 0's 16 bytes.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, SSD_LDS void* ldst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds_addr(ldst))
                 : "memory", "m0");
}
// Bounds-checked forms: offsets at or beyond the record's size read zeros
// (every lane still issues, so the memory-counter arithmetic stays fixed).
__device__ __forceinline__ void dma16_rs(__amdgpu_buffer_rsrc_t rs, uint32_t voff, SSD_LDS void* ldst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(lds_addr(ldst))
                 : "memory", "m0");
}
// Non-temporal forms, for data a workgroup reads exactly once (x rows): they
// leave L2 and the last-level cache to data that is reused.
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t voff, SSD_LDS void* ldst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(base), "s"(lds_addr(ldst))
                 : "memory", "m0");
}
__device__ __forceinline__ void dma16_rs_nt(__amdgpu_buffer_rsrc_t rs, uint32_t voff, SSD_LDS void* ldst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(voff), "s"(rs), "s"(lds_addr(ldst))
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4_rs(__amdgpu_buffer_rsrc_t rs, uint32_t voff, SSD_LDS void* ldst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(lds_addr(ldst))
                 : "memory", "m0");
}
// Raw buffer record over [base, base + bytes) (bytes clamped at 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rs(const void* base, int64_t bytes) {
    const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ void dma4(const void* base, uint32_t voff, SSD_LDS void* ldst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds_addr(ldst))
                 : "memory", "m0");
}

// s_waitcnt vmcnt(n): at most n of this wave's vector-memory operations
// (loads, stores and LDS copies, which retire in order) still outstanding.
// Written with the builtin so that the compiler's own wait insertion knows
// about it (it cannot see inside asm, and would otherwise drain every copy
// in flight before each LDS read).  The builtin is modelled as touching no
// memory, so it is always followed by barrier_lds() or a compiler fence.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) for an n that is a constant once the caller's loop is
// unrolled (the switch folds to one case).
__device__ __forceinline__ void wait_vmcnt_n(int n) {
    switch (n) {
#define SSD_WAIT_CASE(k) case k: wait_vmcnt<k>(); break;
        SSD_WAIT_CASE(0) SSD_WAIT_CASE(1) SSD_WAIT_CASE(2) SSD_WAIT_CASE(3) SSD_WAIT_CASE(4)
        SSD_WAIT_CASE(5) SSD_WAIT_CASE(6) SSD_WAIT_CASE(7) SSD_WAIT_CASE(8) SSD_WAIT_CASE(9)
        SSD_WAIT_CASE(10) SSD_WAIT_CASE(11) SSD_WAIT_CASE(12) SSD_WAIT_CASE(13) SSD_WAIT_CASE(14)
        SSD_WAIT_CASE(15) SSD_WAIT_CASE(16) SSD_WAIT_CASE(17) SSD_WAIT_CASE(18) SSD_WAIT_CASE(19)
        SSD_WAIT_CASE(20) SSD_WAIT_CASE(21) SSD_WAIT_CASE(22) SSD_WAIT_CASE(23) SSD_WAIT_CASE(24)
        SSD_WAIT_CASE(25) SSD_WAIT_CASE(26) SSD_WAIT_CASE(27) SSD_WAIT_CASE(28) SSD_WAIT_CASE(29)
        SSD_WAIT_CASE(30) SSD_WAIT_CASE(31) SSD_WAIT_CASE(32) SSD_WAIT_CASE(33) SSD_WAIT_CASE(34)
        SSD_WAIT_CASE(35) SSD_WAIT_CASE(36) SSD_WAIT_CASE(37) SSD_WAIT_CASE(38) SSD_WAIT_CASE(39)
#undef SSD_WAIT_CASE
        default: wait_vmcnt<0>(); break;
    }
}

// Finish this wave's LDS accesses, then meet the rest of the workgroup.  As
// asm with a "memory" clobber (the s_barrier builtin is modelled as touching
// no memory) so that no LDS access moves across it.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint2 tr16(const SSD_LDS void* p) {
    v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSD_LDS v4s*)p);
    return __builtin_bit_cast(uint2, v);
}

template <typename T>
__device__ __forceinline__ SSD_LDS T* lds(T* p) {
    return (SSD_LDS T*)(p);
}

// Chunk swizzles (16-byte chunk index XOR f(row)).  LDS serves 256 bytes
// per cycle (64 banks x 4 B): a ds_read_b128 takes 16 lanes per cycle and a
// ds_read_b64_tr_b16 32 lanes, so each such lane group must touch 16
// distinct 16-byte bank groups.
// x tiles: 128-byte rows of 64 channels, read only through tr16; the lane
// groups read 4 consecutive rows at 4 chunks each, and rows r and r + 2
// share bank groups unless the second pair moves to the other half-row.
__device__ __forceinline__ int swz_x(int r) { return ((r >> 1) & 1) << 2; }
// B tiles: 256-byte rows of 128 state entries, read as rows (ds_read_b128,
// 16 distinct rows per lane group) by the C.B^T product and through tr16
// (4 consecutive rows at 4 adjacent chunks) by the chunk-state product: a
// bijection of the row's low 4 bits whose upper two bits come from r & 3.
__device__ __forceinline__ int swz_b(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// Hin tiles: 256-byte rows, read as rows in the permuted order of the
// carried-state product (rows {0..7, 16..23} + 8k per lane group).
__device__ __forceinline__ int swz_h(int r) { return (r & 7) | ((r & 16) >> 1); }

// Copy a block of 32 tokens of B (32 rows x 256 B) and x (32 rows x
// 128 B) into one pipeline buffer: 8 + 4 LDS-copy instructions per
// workgroup, spread over its W waves.  Addresses are a wave-uniform base
// (the block's first token) plus a 32-bit per-lane byte offset.  The
// per-lane offsets of whole blocks do not depend on the block and are
// computed once (BxOffsets); a block that runs past the end of the sequence
// re-reads the last token instead (finite values whose weights are zero).
template <int W>
struct BxOffsets {
    uint32_t b[8 / W];
    uint32_t x[4 / W];
};

template <int W>
__device__ __forceinline__ BxOffsets<W> bx_offsets(int wave, int lane, int64_t xstride,
                                                   int64_t bstride) {
    BxOffsets<W> o;
#pragma unroll
    for (int i = 0; i < 8 / W; ++i) {
        const int r = 4 * (wave + i * W) + (lane >> 4);
        o.b[i] = (uint32_t)r * (uint32_t)bstride * 2u + 16u * (uint32_t)((lane & 15) ^ swz_b(r));
    }
#pragma unroll
    for (int i = 0; i < 4 / W; ++i) {
        const int r = 8 * (wave + i * W) + (lane >> 3);
        o.x[i] = (uint32_t)r * (uint32_t)xstride * 2u + 16u * (uint32_t)((lane & 7) ^ swz_x(r));
    }
    return o;
}

template <int W>
__device__ __forceinline__ void issue_bx_stage(int wave, int lane, int tokbase, int L,
                                                 const bf16_t* xbase, int64_t xstride,
                                                 const bf16_t* bbase, int64_t bstride,
                                                 const BxOffsets<W>& off, uint4* bst,
                                                 uint4* xst) {
    // scalar bases are formed here, not hoisted for every future block
    asm volatile("" : "+s"(tokbase));
    if (tokbase + 31 < L) {
        const char* bb = reinterpret_cast<const char*>(bbase + (int64_t)tokbase * bstride);
        const char* xb = reinterpret_cast<const char*>(xbase + (int64_t)tokbase * xstride);
#pragma unroll
        for (int i = 0; i < 8 / W; ++i) dma16(bb, off.b[i], lds(bst) + (wave + i * W) * 64);
#pragma unroll
        for (int i = 0; i < 4 / W; ++i) dma16(xb, off.x[i], lds(xst) + (wave + i * W) * 64);
        return;
    }
    const int tb = min(tokbase, L - 1);
    const char* bb = reinterpret_cast<const char*>(bbase + (int64_t)tb * bstride);
    const char* xb = reinterpret_cast<const char*>(xbase + (int64_t)tb * xstride);
    const uint32_t bs2 = (uint32_t)bstride * 2u, xs2 = (uint32_t)xstride * 2u;
#pragma unroll
    for (int i = 0; i < 8 / W; ++i) {
        const int k = wave + i * W;
        const int r = 4 * k + (lane >> 4);
        const int cc = (lane & 15) ^ swz_b(r);
        const uint32_t dr = (uint32_t)(min(tokbase + r, L - 1) - tb);
        dma16(bb, dr * bs2 + 16u * (uint32_t)cc, lds(bst) + k * 64);
    }
#pragma unroll
    for (int i = 0; i < 4 / W; ++i) {
        const int k = wave + i * W;
        const int r = 8 * k + (lane >> 3);
        const int cc = (lane & 7) ^ swz_x(r);
        const uint32_t dr = (uint32_t)(min(tokbase + r, L - 1) - tb);
        dma16(xb, dr * xs2 + 16u * (uint32_t)cc, lds(xst) + k * 64);
    }
}

// Compile-time replay of one wave's vector-memory issue order, used next to
// each pipelined kernel to check its wait counts: s_waitcnt vmcnt(n) leaves
// at most the n newest operations pending (they complete in issue order), so
// a wait is sound when every operation it guards is older than those n.
struct VmemLog {
    int lab[1024] = {};
    int n = 0;
    int done = 0;   // operations [0, done) are known complete
    constexpr void push(int label, int times) {
        for (int i = 0; i < times; ++i) lab[n++] = label;   // past 1024: not a constant expression
    }
    constexpr bool wait(int count) {   // false if the count does not fit the counter
        if (count < 0 || count > 63) return false;
        if (n - count > done) done = n - count;
        return true;
    }
    // at least one operation carries the label and all of them are complete
    constexpr bool landed(int label) const {
        bool any = false;
        for (int i = 0; i < n; ++i)
            if (lab[i] == label) {
                if (i >= done) return false;
                any = true;
            }
        return any;
    }
};

}  // namespace ssd
