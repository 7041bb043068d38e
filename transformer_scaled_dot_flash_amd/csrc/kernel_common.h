// Internal declarations shared by the HIP kernels and the C ABI layer.
// gfx950 (CDNA4) only: wave64, bf16 MFMA, 160 KiB LDS per workgroup.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Raw buffer resources: 32-bit offsets from an SGPR base, and hardware range
// checking (loads past `num_bytes` return 0, stores past it are dropped).
// Every tensor slice a kernel addresses through one is < 2 GiB (checked on
// the host).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                             0x00020000);
}
__device__ inline u32x4 buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}
// 16-byte load from a buffer straight into LDS: lane i's 16 bytes land at
// lds_block + 16 * i (lds_block is wave-uniform).  Out-of-range lanes write
// zeros.
__device__ inline void buf_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_block, uint32_t byte_off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_block, 16, (int)byte_off, 0, 0, 0);
}
// The same with the non-temporal cache hint (nt), for data read exactly
// once (a decode step's K/V cache): the stream then does not displace
// reused lines in L2 and the Infinity Cache (measured +9% on the decode).
__device__ inline void buf_load_lds16_nt(__amdgpu_buffer_rsrc_t r, void* lds_block, uint32_t byte_off) {
    constexpr int kNonTemporal = 2;  // cache-policy bit nt
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_block, 16, (int)byte_off, 0, 0, kNonTemporal);
}
// Byte address of an LDS object (the 32-bit offset LDS instructions take).
__device__ inline uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Transposing LDS read (ds_read_b64_tr_b16) of lds_addr + OFF.  Within each
// group of 16 lanes, source lane r points at 4 consecutive bf16 values
// R[r][0..3]; destination lane i receives R[i/4 + 4k][i%4] for k = 0..3.
//
// Issued as inline assembly on purpose: for the compiler's own intrinsic the
// compiler cannot tell the read apart from the LDS written by outstanding
// buffer-to-LDS loads and puts a full vmcnt(0) wait in front of it, which
// stalls every wave until all of its tile prefetches have landed.  The
// compiler does not track this read, so its result may only be used after
// lds_wait_bind; the "memory" clobber keeps it in program order with every
// other memory access.
template <int OFF>
__device__ inline bf16x4 ds_read_tr16_asm(uint32_t lds_addr) {
    static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS offset");
    bf16x4 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "n"(OFF) : "memory");
    return r;
}

// ds_read_b128 as inline assembly, for reads that must stay in flight a
// fixed distance ahead of their use (the compiler's scheduler sinks
// intrinsic reads next to their first use when registers are tight).  Same
// contract as ds_read_tr16_asm: the result may only be used after a wait
// that binds it (lds_wait_bind1).
template <int OFF>
__device__ inline bf16x8 ds_read_b128_asm(uint32_t lds_addr) {
    static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS offset");
    bf16x8 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "n"(OFF) : "memory");
    return r;
}

// s_waitcnt lgkmcnt(N) binding one 16-byte fragment (see lds_wait_bind).
template <int N>
__device__ inline void lds_wait_bind1(bf16x8& f) {
    static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(f) : "n"(N));
}

// s_waitcnt lgkmcnt(N) that also redefines the fragments f, so no use of f
// can be scheduled before it.  LDS operations complete in issue order, so
// once at most N are outstanding, every read issued before the last N has
// completed (other LDS or scalar operations only make the wait stricter).
template <int N, int ND>
__device__ inline void lds_wait_bind(bf16x4 (&f)[2][ND]) {
    static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
    static_assert(ND == 2 || ND == 4, "two or four 32-feature blocks");
    if constexpr (ND == 4)
        asm volatile("s_waitcnt lgkmcnt(%8)"
                     : "+v"(f[0][0]), "+v"(f[0][1]), "+v"(f[0][2]), "+v"(f[0][3]), "+v"(f[1][0]),
                       "+v"(f[1][1]), "+v"(f[1][2]), "+v"(f[1][3])
                     : "n"(N));
    else
        asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(f[0][0]), "+v"(f[0][1]), "+v"(f[1][0]), "+v"(f[1][1]) : "n"(N));
}

// O^T += V^T P^T over one V tile in LDS (row-major, swizzled by swz), for
// RB blocks of 32 query columns.  Lane (feature d, half hi) needs V for the
// keys 16ks + 4hi + {0..3} and 16ks + 8 + 4hi + {0..3} that its P operand
// (the score accumulator layout) holds; two transposing reads per 32-feature
// block deliver exactly those.  va[h][db] is the lane's address of key step 0
// for the low (h = 0) and high (h = 1) key group of feature block db; key step
// ks adds 16 rows.  The reads of step ks + 1 are in flight while the MFMAs
// of step ks run; each V fragment feeds RB MFMAs.
template <int KS, int D>
__device__ inline void pv_issue(bf16x4 (&f)[2][D / 32], const uint32_t (&va)[2][D / 32]) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        f[0][db] = ds_read_tr16_asm<KS * 16 * D * 2>(va[0][db]);
        f[1][db] = ds_read_tr16_asm<KS * 16 * D * 2>(va[1][db]);
    }
}
template <int KS, int D, int NKS, int RB>
__device__ inline void pv_step(f32x16 (&oacc)[RB][D / 32], const bf16x8 (&pb)[RB][NKS],
                               bf16x4 (&cur)[2][D / 32], bf16x4 (&nxt)[2][D / 32],
                               const uint32_t (&va)[2][D / 32]) {
    constexpr bool more = KS + 1 < NKS;
    if constexpr (more) pv_issue<KS + 1, D>(nxt, va);
    lds_wait_bind<more ? 2 * (D / 32) : 0, D / 32>(cur);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const bf16x8 a = {cur[0][db][0], cur[0][db][1], cur[0][db][2], cur[0][db][3],
                          cur[1][db][0], cur[1][db][1], cur[1][db][2], cur[1][db][3]};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[rb][KS], oacc[rb][db], 0, 0, 0);
    }
}
template <int D, int NKS, int RB, int... KS>
__device__ inline void pv_steps(f32x16 (&oacc)[RB][D / 32], const bf16x8 (&pb)[RB][NKS],
                                bf16x4 (&f)[2][2][D / 32], const uint32_t (&va)[2][D / 32],
                                std::integer_sequence<int, KS...>) {
    (pv_step<KS, D, NKS, RB>(oacc, pb, f[KS & 1], f[(KS + 1) & 1], va), ...);
}
// NKS key steps of 16 keys: the whole tile.
template <int D, int NKS, int RB>
__device__ inline void pv_tile(f32x16 (&oacc)[RB][D / 32], const bf16x8 (&pb)[RB][NKS],
                               const uint32_t (&va)[2][D / 32]) {
    bf16x4 f[2][2][D / 32];
    pv_issue<0, D>(f[0], va);
    pv_steps<D, NKS, RB>(oacc, pb, f, va, std::make_integer_sequence<int, NKS>{});
}
// Wait until at most N vector-memory operations of this wave are in flight
// (s_waitcnt vmcnt(N)), leaving the LDS/scalar and export counters
// unconstrained.  gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] << 14.
template <int N>
__device__ inline void wait_vmem_le() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ inline void wait_vmem_all() { wait_vmem_le<0>(); }

// Value of lane (lane ^ 32), through the LDS crossbar (no memory access).
// `addr` = 4 * (lane ^ 32), computed once per kernel.
__device__ inline float swap_halves(float x, int addr) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x)));
}

// Layout of K and V tiles in LDS: row-major, 16-byte chunk c of row `key`
// stored at chunk c ^ swz(key).  gfx950 LDS has 64 banks of 4 bytes (256 B
// per clock).  The swizzle makes both read patterns conflict-free:
//   * MFMA K reads, ds_read_b128 (16 lanes per clock): 16 consecutive keys,
//     one logical chunk -> 16 distinct physical chunks;
//   * transposing V reads, ds_read_b64_tr_b16 (32 lanes per clock): 4
//     consecutive keys (aligned to 4) x 4 adjacent chunks -> 16 distinct
//     bank groups.
// With 256-byte rows (D = 128) every row starts at bank 0, so swz is a
// bijection on 4 bits that moves the key's low 2 bits to the chunk's high
// 2 bits.  With 128-byte rows (D = 64) odd rows start at bank 32, and the
// 3-bit swizzle only has to separate keys of equal parity.
template <int CPR>
__device__ inline int swz(int key) {
    if (CPR == 16) return ((key & 3) << 2) | ((key >> 2) & 3);
    return (((key >> 1) & 1) << 2) | ((key >> 2) & 3);
}

// Lane offsets (bytes, within a V tile) of the transposing reads of key step
// 0 used by pv_tile.  swz only depends on the low 4 bits of the key, so key
// step ks is these offsets plus 16 rows.
template <int D>
__device__ inline void pv_lane_offsets(uint32_t (&voff)[2][D / 32], int lane) {
    constexpr int CPR = D / 8;
    const int i = lane & 15;
    const int key = 4 * (lane >> 5) + (i >> 2);
    const int d = 16 * ((lane >> 4) & 1) + 4 * (i & 3);  // feature within a 32-block
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int k = key + 8 * h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            voff[h][db] = (uint32_t)(k * D * 2 + (d & 7) * 2 + (((db * 4 + (d >> 3)) ^ swz<CPR>(k)) * 16));
    }
}
__device__ inline void buf_store_b64(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)byte_off, 0, 0);
}
__device__ inline void buf_store_b128(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_off, 0, 0);
}

// log2(e): the kernels evaluate exp(x) as exp2(x * log2 e) and fold the
// factor into the score multiplier once on the host.
constexpr double kLog2e = 1.4426950408889634073599246810019;

// Paged KV cache of the decode kernel (block_table == nullptr: contiguous).
struct PagedKV {
    const int* block_table;  // [B][max_pages] physical page of each logical page
    const int* seq_lens;     // [B] keys of each sequence
    int max_pages;           // columns of block_table
    int page_shift;          // log2(page_size)
    int num_pages;           // pages in each pool
};

}  // namespace attn
