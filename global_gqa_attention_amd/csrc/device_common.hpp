// device_common.hpp -- small gfx950 building blocks shared by the attention kernels.
//
// MFMA lane layouts used throughout (checked on gfx950 for v_mfma_f32_32x32x16_bf16):
//   A operand (32 x 16): lane l holds row l % 32, k = 8 * (l / 32) + t for t = 0..7
//   B operand (16 x 32): lane l holds column l % 32, k = 8 * (l / 32) + t
//   C / D     (32 x 32): lane l holds column l % 32, slot j = row 8 * (j / 4) + 4 * (l / 32) + j % 4
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mimo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int DQK = 192;    // Q/K head width
constexpr int DVV = 128;    // V head width
constexpr int NHALF = 32;   // rotary pairs: dims (d, d + 32) for d < 32; 64 rotated dims in all
constexpr float VSCALE = 0.707f;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }
__device__ __forceinline__ __bf16 f2bf(float x) { return (__bf16)x; }  // round to nearest even

__device__ __forceinline__ bf16x8 ld16(const u16 *p) { return __builtin_bit_cast(bf16x8, *(const uint4 *)p); }
__device__ __forceinline__ uint4 ldu4(const u16 *p) { return *(const uint4 *)p; }
__device__ __forceinline__ void st16(u16 *p, bf16x8 x) { *(uint4 *)p = __builtin_bit_cast(uint4, x); }
__device__ __forceinline__ void st16u(u16 *p, uint4 x) { *(uint4 *)p = x; }
// Non-temporal (streaming) forms, for data that a kernel reads or writes exactly once: those lines then do
// not displace reused ones in the caches (the D/LSE pass, which streams O and dO, runs 19% faster so).
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldu4_nt(const void *p) { return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const nt_u32x4 *)p)); }
__device__ __forceinline__ bf16x8 ld16_nt(const u16 *p) { return __builtin_bit_cast(bf16x8, ldu4_nt(p)); }
__device__ __forceinline__ void st16u_nt(u16 *p, uint4 x) { __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4, x), (nt_u32x4 *)p); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Values of lanes l and l ^ 32 combined: v_permlane32_swap gives every lane the lower-half value in .x and
// the upper-half value in .y of its pair.
__device__ __forceinline__ float pair_max(float v)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((address_space(3))) void lds_void;

// Direct HBM -> LDS copy of 16 bytes per lane: lane i's bytes land at lds_wave_base + 16 i (lds_wave_base
// must be wave-uniform).  Issued through inline asm so that the compiler adds no automatic wait for it
// before later LDS reads; the caller orders it with wait_vmcnt<N>() and barriers.  It has no register
// output, so nothing can be overwritten by the load in flight.
__device__ __forceinline__ void lds_dma16(const void *gsrc, void *lds_wave_base)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void *)lds_wave_base;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(m0), "v"(gsrc)
                 : "memory", "m0");
}

// The same copy from a wave-uniform base address plus a per-lane byte offset (saddr form: the per-lane
// part needs no 64-bit address arithmetic).
__device__ __forceinline__ void lds_dma16(const void *sbase, uint32_t voff, void *lds_wave_base)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void *)lds_wave_base;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

// The saddr copy with the LDS destination given as its 32-bit LDS address (the m0 value itself).
__device__ __forceinline__ void lds_dma16_m0(const void *sbase, uint32_t voff, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

// The per-lane-address copy with the non-temporal hint, for data read once.
__device__ __forceinline__ void lds_dma16_nt(const void *gsrc, void *lds_wave_base)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void *)lds_wave_base;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :
                 : "s"(m0), "v"(gsrc)
                 : "memory", "m0");
}

// The same with the non-temporal hint, for data read once (keeps it from displacing reused lines in L2).
__device__ __forceinline__ void lds_dma16_nt(const void *sbase, uint32_t voff, void *lds_wave_base)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void *)lds_wave_base;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(m0), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory loads are still in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS swizzles for tiles filled by lds_dma16: the position of logical 16-byte chunk q in row r of a tile
// whose rows are 384, 256, 128 or 64 bytes long.  gfx950 serves a 16-byte-per-lane LDS read 16 lanes at a
// time from 64 banks; an MFMA operand read has 16 consecutive lanes on 16 consecutive rows at one logical
// chunk, and each mapping sends those 16 reads to 16 different 16-byte bank groups.  Each is an
// involution, so it also maps a position back to its logical chunk.
__device__ __forceinline__ int swz384(int r, int q) { return (q & ~7) | ((q & 7) ^ ((r >> 1) & 7)); }
__device__ __forceinline__ int swz256(int r, int q) { return q ^ (r & 15); }
__device__ __forceinline__ int swz128(int r, int q) { return q ^ ((r >> 1) & 7); }
__device__ __forceinline__ int swz64(int r, int q) { return q ^ ((r >> 2) & 3); }
// Swizzles for tiles that are also read transposed with ds_read_b64_tr_b16 (16 lanes read 4 consecutive
// rows x 4 consecutive chunk halves; a half-wave of such reads must cover all 64 banks once): the XOR
// term moves rows r and r + 2 into different 4-chunk groups while keeping the 16-row row reads above
// conflict-free.  384-byte rows (24 chunks, XOR inside groups of 8) and 256-byte rows.
__device__ __forceinline__ int swz384t(int r, int q) { return (q & ~7) | ((q & 7) ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))); }
__device__ __forceinline__ int swz256t(int r, int q) { return q ^ ((4 * (r & 3) + ((r >> 2) & 3)) & 15); }

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of the 4-element row read
// by lane 4 t + i / 4 as its element t.  Two such reads give an 8-element MFMA operand.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 ld_tr(const void *lds_addr)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(lds_void *)lds_addr);
}
__device__ __forceinline__ bf16x8 tr_pair(const char *p0, const char *p1)
{
    const s16x4 x = ld_tr(p0), y = ld_tr(p1);
    const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
    return __builtin_bit_cast(bf16x8, make_uint4(ux.x, ux.y, uy.x, uy.y));
}

// THD work items: sequence b (bounds cu[b] .. cu[b + 1]) holds count(start, end) items, numbered from the
// last sequence backwards (item 0 is the last sequence's item 0).  Returns the sequence holding item idx,
// its bounds and the item's index inside it (b = -1 past the last item); all wave-uniform.  The lanes read
// cu_seqlens in parallel (one load per 64 sequences) and a wave prefix sum locates the item, instead of a
// chain of dependent loads, one per sequence.
struct SeqPos {
    int b, start, end, j;
};
template <typename Count>
__device__ __forceinline__ SeqPos seq_lookup_rev(const int *cu, int batch, int idx, Count count)
{
    const int lane = threadIdx.x & 63;
    int before = 0;   // items of the sequences already passed
    for (int c0 = 0; c0 < batch; c0 += 64) {
        const int b = batch - 1 - (c0 + lane);
        int s = 0, e = 0, n = 0;
        if (b >= 0) {
            s = cu[b];
            e = cu[b + 1];
            n = count(s, e);
        }
        int incl = n;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        const unsigned long long hit = __ballot(before + incl > idx);
        if (hit) {
            const int L = __builtin_ctzll(hit);
            SeqPos r;
            r.b = __builtin_amdgcn_readlane(b, L);
            r.start = __builtin_amdgcn_readlane(s, L);
            r.end = __builtin_amdgcn_readlane(e, L);
            r.j = idx - before - (__builtin_amdgcn_readlane(incl, L) - __builtin_amdgcn_readlane(n, L));
            return r;
        }
        before += __builtin_amdgcn_readlane(incl, 63);
    }
    return SeqPos{-1, 0, 0, 0};
}

// Rotate-half RoPE of one 8-wide chunk pair: x0 holds dims d..d+7 (d < 32), x1 dims d+32..d+39, cs the
// (cos, sin) of the 8 matching frequencies.  Rounded back to bf16 (the MFMA operand precision).
__device__ __forceinline__ void rope_pair(bf16x8 &x0, bf16x8 &x1, const float2 *cs)
{
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        float a = bf2f(x0[t]), b = bf2f(x1[t]);
        float c = cs[t].x, s = cs[t].y;
        x0[t] = f2bf(a * c - b * s);
        x1[t] = f2bf(b * c + a * s);
    }
}

}  // namespace mimo
