// Staging of 16-bit (bf16 or fp16) [rows x D] tiles from HBM into row-major LDS tiles for the
// MFMA kernels, plus the operand-read helpers that work on those tiles.
//
// gfx950 LDS has 128 four-byte banks.  Measured on MI355X: a 16-byte-per-lane read serves 32
// lanes per cycle, and an 8-byte transpose read (ds_read_b64_tr_b16) 64 lanes; row strides
// are padded so that the rows a read touches in one cycle fall on distinct banks.  An MFMA
// whose contraction runs over rows (keys or queries) takes one operand straight from an
// earlier accumulator; the other operand, whose rows must be in the accumulator's row order,
// comes from the same row-major tile through transpose reads, so no transposed copy of any
// tile is ever stored.
#pragma once

#include "common.h"

namespace fa {

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes return zero
// without touching memory, which zero-fills rows past T with no branch.  Descriptor word 3
// is the gfx9-family raw-buffer format.
struct Buf {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ Buf(const void* base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                              0x00020000)) {}
    __device__ __forceinline__ u32x4 load16(uint32_t off) const {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    }
};

// Buffer over rows [0, T) of one head: rows of D 16-bit elements, `ld` elements apart
// (ld >= D).  It ends with the last row's D elements, so reads at rows past T return zeros
// whatever the layout puts there.
template <int D>
__device__ __forceinline__ Buf head_buf(const uint16_t* base, int64_t ld, int T) {
    return Buf(base, (uint32_t)(((int64_t)(T - 1) * ld + D) * 2));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 32-bit LDS address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// The same address, opaque to the compiler: it stays in one register as computed, instead of
// being rebuilt from its parts by a vector add in every loop iteration (which the compiler
// does for addresses it can recompute, to save a register).
__device__ __forceinline__ uint32_t pinned_lds_addr(uint32_t a) {
    asm volatile("" : "+v"(a));
    return a;
}

// Typed loads at a 32-bit LDS address (constant displacements fold into the instruction's
// offset field).
template <class T>
__device__ __forceinline__ T lds_load(uint32_t a) {
    return *(const __attribute__((address_space(3))) T*)(a);
}
template <class E>
__device__ __forceinline__ typename E::v4 lds_load_tr4(uint32_t a) {
    typedef __bf16 v4bf16 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(typename E::v4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                  (__attribute__((address_space(3))) v4bf16*)(a)));
}

// s_waitcnt vmcnt(N) only (gfx9 encoding: vmcnt in [3:0] and [15:14]; expcnt [6:4] and
// lgkmcnt [11:8] left at their "no wait" maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that does not also wait for outstanding vector-memory loads (which
// __syncthreads() does); the memory clobber keeps the compiler from moving LDS accesses
// across it.  Data written to LDS by a wave's LDS-DMA loads is visible to the other waves
// after the barrier once that wave has waited for those loads (wait_vmcnt).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Padded row-major [rows x D] 16-bit tile filled by LDS-DMA: rows are D + 8*PADC elements
// apart.  Measured on gfx950 (128 banks, 32 lanes serviced together): 16-byte reads of 32
// consecutive rows at one chunk are conflict-free at D + 8 and D + 24 (an odd number of
// 16-byte slots per row whose product with 16 rows is not a multiple of the 512-byte bank
// line) but 2-way conflicted at D + 16 and 16-way at D; transpose reads of 8 rows x 32 bytes
// are conflict-free at D + 16 and D + 24 but 2-way at D and D + 8.  The 16x16x32 operand
// pattern, 16-byte reads of 16 consecutive rows at two adjacent chunks per 32 lanes, and
// transpose reads of 4 rows x 32 bytes per 16 lanes are both conflict-free at D + 16 (the 16
// rows' 32-byte pieces then tile the 128 banks) and conflicted at D + 8 and D + 24.
// Slot s (16 bytes) of the tile is row s / (CPR + PADC), chunk s % (CPR + PADC);
// a pad slot receives a copy of the row's last chunk, so every lane loads valid bytes.
template <int D, int PADC = 1>
struct Pad {
    static constexpr int CPR = D / 8;               // data chunks per row
    static constexpr int SPR = CPR + PADC;          // slots per row
    static constexpr int ROWB = 16 * SPR;           // bytes per row
};
template <int D, int PADC = 1>
__device__ __forceinline__ uint32_t dma_src_offset_padded(int p, int lane, uint32_t ld_bytes) {
    using P = Pad<D, PADC>;
    const int slot = p * 64 + lane;
    const int r = slot / P::SPR;
    int cch = slot % P::SPR;
    if (cch >= P::CPR) cch = P::CPR - 1;
    return (uint32_t)r * ld_bytes + 16u * (uint32_t)cch;
}

// LDS-DMA of 64 lanes x 4 bytes (256 consecutive LDS bytes at `dst`).
__device__ __forceinline__ void dma_dwords(const Buf& src, void* dst, uint32_t voff, int soff) {
    const uint32_t lds = (uint32_t)(uintptr_t)(lds_ptr_t)dst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(src.r), "s"(soff)
                 : "memory", "m0");
}

// One LDS-DMA piece: 64 lanes x 16 bytes from `src` (voffset per lane, soffset uniform)
// into the 1 KB of LDS at `dst` (wave-uniform).  Issued from asm: the compiler then adds no
// implicit waits for it (it cannot tell which LDS reads it may alias and would wait for
// every outstanding load before them); the kernels order it explicitly with wait_vmcnt
// and lds_barrier.  M0 carries the LDS address; one wait state after writing it.
__device__ __forceinline__ void dma_piece(const Buf& src, void* dst, uint32_t voff, int soff) {
    const uint32_t lds = (uint32_t)(uintptr_t)(lds_ptr_t)dst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(src.r), "s"(soff)
                 : "memory", "m0");
}

// Work item (query tile, b, h) of a workgroup id for query-tile-major kernels: longest key
// ranges (last query tiles) first; with GQA (xcd_group), the rep query heads of a KV head
// get ids congruent mod 8, so the round-robin dispatcher puts them on one XCD together.
__device__ __forceinline__ void decode_q_work(int id, int nqt, int B, int H, int HKV,
                                              int xcd_group, int& qt, int& b, int& h) {
    int rank;
    if (xcd_group) {
        const int rep = H / HKV;
        const int hig = (id >> 3) % rep;
        const int rest = (id / (8 * rep)) * 8 + (id & 7);
        rank = rest / (B * HKV);
        const int grp = rest % (B * HKV);
        b = grp / HKV;
        h = (grp % HKV) * rep + hig;
    } else {
        rank = id / (B * H);
        const int bh = id % (B * H);
        b = bh / H;
        h = bh % H;
    }
    qt = nqt - 1 - rank;
}

// max over an accumulator tile without NaN canonicalisation (v_maximum3_f32)
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// A operand (M = 16 columns c0 .. c0 + 15 of a row-major tile, K = 32 rows) of a 16x16x32
// MFMA whose B operand comes from 16x16 accumulators: lane l = 16g + j covers column c0 + j,
// and element e holds row r0 + 4g + e (e < 4) or r0 + 16 + 4g + e - 4 -- the rows in which
// lane row g of two stacked 16-row accumulator tiles holds its entries.  Two LDS transpose
// reads of 4 rows each: the 16 lanes of row g address rows r0 + 4g + j/4 at columns
// c0 + 4*(j%4) .. +3, and lane j receives column c0 + j of the four rows.
template <class E, int LD>
__device__ __forceinline__ typename E::v8 tr_operand16(const uint16_t* tile, int r0, int c0, int lane) {
    const int j = lane & 15, g = lane >> 4;
    const uint16_t* p = tile + (r0 + 4 * g + (j >> 2)) * LD + c0 + 4 * (j & 3);
    const typename E::v4 lo = lds_read_tr4e<E>(p);
    const typename E::v4 hi = lds_read_tr4e<E>(p + 16 * LD);
    typename E::v8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = lo[e];
        r[4 + e] = hi[e];
    }
    return r;
}

inline int xcd_group_for(int nqt, int B, int H, int HKV) {
    const int rep = H / HKV;
    return (rep > 1 && ((long)nqt * B * HKV) % 8 == 0) ? 1 : 0;
}

}  // namespace fa
