// attn_append.hip -- write new tokens into a paged KV cache (gfx950).
//
// Token i's key is rotated at positions[i] (RoPE on dims 0..63, rotate-half pairs (d, d+32), angle
// p * base^(-d/32); the angles in fp64, cos/sin rounded to fp32, the rotation in fp32, bf16
// round-to-nearest-even: the same values the forward's key preparation produces) and stored with its
// unscaled value in pool row slots[i] (page size 1: one token per row).  Source: SGLang cookbook page
// "MiMo-V2.6", section 2 "Configuration tips", "Context length and memory" (page size 1); miles docs
// "MiMo-V2.6-Flash" section 1 (partial RoPE on 64 of 192 dims, RoPE bases).
#include "device_common.hpp"
#include "internal.hpp"

namespace mimo {
namespace {

// One workgroup of 64 threads per (token, KV head): threads 0..31 compute the angle of dim t once (fp64),
// threads 0..3 then rotate K chunk pairs (c, c + 4) with the eight (cos, sin) they fetch by lane shuffles,
// threads 4..19 copy K chunks 8..23, threads 20..35 copy the 16 V chunks.  Slots outside the pool are
// skipped.
__global__ __launch_bounds__(64) void cache_append_kernel(const uint16_t *k, const uint16_t *v, const int32_t *positions,
                                                          const int32_t *slots, int hkv, int pool_rows, double base,
                                                          uint16_t *k_pool, uint16_t *v_pool)
{
    const int i = blockIdx.x, kvh = blockIdx.y, t = threadIdx.x;
    const int slot = slots[i];
    if (slot < 0 || slot >= pool_rows) return;
    const u16 *ks = k + ((size_t)i * hkv + kvh) * DQK;
    u16 *kd = k_pool + ((size_t)slot * hkv + kvh) * DQK;
    float cf = 0.f, sf = 0.f;
    {
        const double ang = (double)positions[i] * pow(base, -(double)(t & 31) / (double)NHALF);
        double sn, cn;
        sincos(ang, &sn, &cn);
        cf = (float)cn;
        sf = (float)sn;
    }
    float2 cs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cs[e] = make_float2(__shfl(cf, 8 * (t & 3) + e, 64), __shfl(sf, 8 * (t & 3) + e, 64));
    if (t < 4) {
        bf16x8 x0 = ld16(ks + 8 * t), x1 = ld16(ks + 8 * (t + 4));
        rope_pair(x0, x1, cs);
        st16(kd + 8 * t, x0);
        st16(kd + 8 * (t + 4), x1);
    } else if (t < 20) {
        const int ch = t + 4;                       // chunks 8..23
        st16u(kd + 8 * ch, ldu4(ks + 8 * ch));
    } else if (t < 36) {
        const int ch = t - 20;
        st16u(v_pool + ((size_t)slot * hkv + kvh) * DVV + 8 * ch, ldu4(v + ((size_t)i * hkv + kvh) * DVV + 8 * ch));
    }
}

}  // namespace

hipError_t launch_cache_append(const uint16_t *k, const uint16_t *v, const int32_t *positions, const int32_t *slots,
                               int n, int hkv, int pool_rows, double rope_base, uint16_t *k_pool, uint16_t *v_pool,
                               hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    trace_begin("cache_append", stream);
    cache_append_kernel<<<dim3((unsigned)n, (unsigned)hkv), 64, 0, stream>>>(k, v, positions, slots, hkv, pool_rows,
                                                                             rope_base, k_pool, v_pool);
    trace_end(stream);
    return hipGetLastError();
}

}  // namespace mimo
