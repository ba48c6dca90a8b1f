// attn_prep.hip -- per-call K/V preparation for the attention kernels (gfx950).
//
// Writes two workspace tensors that let the hot loops move K and V from HBM straight into LDS with
// global_load_lds (no register staging, no per-tile arithmetic):
//   kr [T_pad, hkv, 192] bf16: k with RoPE applied to dims 0..63 at each token's position inside its own
//                              sequence (rotate-half pairs (d, d+32), angle p * base^(-d/32)), i.e. the k'
//                              of miles docs "MiMo-V2.6-Flash" section 1 (partial RoPE on 64 of 192 dims);
//   vt [hkv, 128, T_pad] bf16: v transposed per KV head, with the 4-token chunks of every 16-token group
//                              stored in the order (0, 2, 1, 3): an MFMA operand read of 8 consecutive
//                              elements then returns the keys in the order the score registers hold them.
// Tokens T .. T_pad-1 are written as zeros (tiles may read them; they are masked, and zero values keep the
// masked products finite).  For a prefill over a cached prefix the same two tensors cover one key stream
// per sequence: its cache rows (K already rotated), then its new tokens.
#include "device_common.hpp"
#include "internal.hpp"

namespace mimo {
namespace {

constexpr int PT = 64;   // tokens per workgroup

__device__ __forceinline__ int seq_start_of(const int32_t *cu, int batch, int t)
{
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return cu[lo];
}

__device__ __forceinline__ int vperm16(int t)   // column of token t inside its 16-token group
{
    const int c4 = (t >> 2) & 3;
    return (t & ~15) | ((((c4 & 1) << 1) | (c4 >> 1)) << 2) | (t & 3);
}

__global__ __launch_bounds__(256) void kv_prep_kernel(const LayerArgs a, KVPrep p)
{
    __shared__ __attribute__((aligned(16))) u16 sV[PT * (DVV + 8)];
    const int tid = threadIdx.x;
    const int kvh = blockIdx.x % a.hkv;            // KV head fastest: a token's heads are one contiguous run
    const int t0 = (blockIdx.x / a.hkv) * PT;

    // ---- K: token t0 + tid/4, chunk group tid%4 (chunks cg, cg+4 rotated; 8+cg+4i copied)
    {
        const int t = t0 + (tid >> 2), cg = tid & 3;
        u16 *dst = p.kr + ((size_t)t * a.hkv + kvh) * DQK;
        if (t < a.T) {
            const u16 *src = a.k + ((size_t)t * a.hkv + kvh) * DQK;
            bf16x8 x0 = ld16_nt(src + 8 * cg), x1 = ld16_nt(src + 8 * (cg + 4));
            const int pos = t - seq_start_of(a.cu, a.batch, t);
            const float2 *cs = a.rope + (size_t)min(pos, a.rope_len - 1) * NHALF + 8 * cg;
            float2 c8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c8[i] = cs[i];
            rope_pair(x0, x1, c8);
            uint4 rest[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) rest[i] = ldu4_nt(src + 8 * (8 + cg + 4 * i));
            st16(dst + 8 * cg, x0);
            st16(dst + 8 * (cg + 4), x1);
#pragma unroll
            for (int i = 0; i < 4; ++i) st16u(dst + 8 * (8 + cg + 4 * i), rest[i]);
            if (p.k_rot) {   // the rotated rows once more, for the backward
                u16 *kd = p.k_rot + ((size_t)t * a.hkv + kvh) * DQK;
                st16u_nt(kd + 8 * cg, __builtin_bit_cast(uint4, x0));
                st16u_nt(kd + 8 * (cg + 4), __builtin_bit_cast(uint4, x1));
#pragma unroll
                for (int i = 0; i < 4; ++i) st16u_nt(kd + 8 * (8 + cg + 4 * i), rest[i]);
            }
        } else if (t < p.T_pad) {
            const uint4 z = make_uint4(0, 0, 0, 0);
            st16u(dst + 8 * cg, z);
            st16u(dst + 8 * (cg + 4), z);
#pragma unroll
            for (int i = 0; i < 4; ++i) st16u(dst + 8 * (8 + cg + 4 * i), z);
        }
    }
    // ---- V^T: stage 64 tokens x 128 dims in LDS, then write rows of 8 tokens (permuted order)
    {
        const int r = tid >> 2, cg = tid & 3;
        const int t = t0 + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = cg + 4 * i;
            uint4 x = make_uint4(0, 0, 0, 0);
            if (t < a.T) x = ldu4_nt(a.v + ((size_t)t * a.hkv + kvh) * DVV + 8 * ch);
            *(uint4 *)(sV + r * (DVV + 8) + 8 * ch) = x;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int item = tid + 256 * i;          // 128 dims x 8 column chunks
        const int d = item >> 3, cc = item & 7;  // cc: columns 8cc..8cc+7 of the tile
        if (t0 + 8 * cc >= p.T_pad) continue;
        bf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // column 8cc+e holds the token whose permuted column is 8cc+e (the permutation is an involution)
            const int tok = vperm16(8 * cc + e);
            w[e] = __builtin_bit_cast(__bf16, sV[tok * (DVV + 8) + d]);
        }
        st16(p.vt + ((size_t)kvh * DVV + d) * p.T_pad + t0 + 8 * cc, w);
    }
}

// Sequence b of the combined key stream (cache rows, then new tokens) that holds key index u: the b with
// cu_cache[b] + cu[b] <= u < cu_cache[b+1] + cu[b+1].
__device__ __forceinline__ int seq_of_keys(const int32_t *cu, const int32_t *cuc, int batch, int u)
{
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cuc[mid] + cu[mid] <= u) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// The same layout as kv_prep_kernel over the combined key stream of a cached prefill: key u of sequence b
// is cache row cu_cache[b] + j (already rotated: copied) for j = u - (cu_cache[b] + cu[b]) < n_b, else new
// token cu[b] + j - n_b, rotated at position positions[b] + j - n_b.
__global__ __launch_bounds__(256) void kv_prep_cached_kernel(const LayerArgs a, KVPrep p, const CacheArgs C)
{
    __shared__ __attribute__((aligned(16))) u16 sV[PT * (DVV + 8)];
    const int tid = threadIdx.x;
    const int kvh = blockIdx.x % a.hkv;            // KV head fastest: a token's heads are one contiguous run
    const int t0 = (blockIdx.x / a.hkv) * PT;
    const int Tk = a.T + C.Tc;
    // source rows of key u: (K row, V row, rotation position or -1 for a cache row).  Returns false when the
    // index arrays do not account for key u (their totals disagree with T and Tc): the key is then zero-filled
    // instead of read from outside the tensors.
    auto source = [&](int u, const u16 *&ks, const u16 *&vs, int &pos) {
        const int b = seq_of_keys(a.cu, C.cu_cache, a.batch, u);
        const int j = u - (C.cu_cache[b] + a.cu[b]);
        const int n = C.cu_cache[b + 1] - C.cu_cache[b];
        if (j < n) {
            const int cr = C.cu_cache[b] + j;
            if (cr < 0 || cr >= C.Tc) return false;
            const size_t row = (size_t)(C.page_table ? C.page_table[cr] : cr) * a.hkv + kvh;
            ks = C.k_cache + row * DQK;
            vs = C.v_cache + row * DVV;
            pos = -1;
        } else {
            const int t = a.cu[b] + j - n;
            if (t < 0 || t >= a.T) return false;
            const size_t row = (size_t)t * a.hkv + kvh;
            ks = a.k + row * DQK;
            vs = a.v + row * DVV;
            pos = max(C.positions[b] + j - n, 0);
        }
        return true;
    };

    // ---- K: key t0 + tid/4, chunk group tid%4 (chunks cg, cg+4 rotated for new tokens; 8+cg+4i copied)
    {
        const int u = t0 + (tid >> 2), cg = tid & 3;
        u16 *dst = p.kr + ((size_t)u * a.hkv + kvh) * DQK;
        const u16 *src = nullptr, *vs = nullptr;
        int pos = 0;
        if (u < Tk && source(u, src, vs, pos)) {
            bf16x8 x0 = ld16_nt(src + 8 * cg), x1 = ld16_nt(src + 8 * (cg + 4));
            if (pos >= 0) {
                const float2 *cs = a.rope + (size_t)min(pos, a.rope_len - 1) * NHALF + 8 * cg;   // pos >= 0 here
                float2 c8[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) c8[i] = cs[i];
                rope_pair(x0, x1, c8);
            }
            st16(dst + 8 * cg, x0);
            st16(dst + 8 * (cg + 4), x1);
#pragma unroll
            for (int i = 0; i < 4; ++i) st16u(dst + 8 * (8 + cg + 4 * i), ldu4_nt(src + 8 * (8 + cg + 4 * i)));
        } else if (u < p.T_pad) {
            const uint4 z = make_uint4(0, 0, 0, 0);
            st16u(dst + 8 * cg, z);
            st16u(dst + 8 * (cg + 4), z);
#pragma unroll
            for (int i = 0; i < 4; ++i) st16u(dst + 8 * (8 + cg + 4 * i), z);
        }
    }
    // ---- V^T: stage 64 keys x 128 dims in LDS, then write rows of 8 keys (permuted order)
    {
        const int r = tid >> 2, cg = tid & 3;
        const int u = t0 + r;
        const u16 *ks = nullptr, *vs = nullptr;
        int pos = 0;
        const bool have = u < Tk && source(u, ks, vs, pos);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = cg + 4 * i;
            uint4 x = make_uint4(0, 0, 0, 0);
            if (have) x = ldu4_nt(vs + 8 * ch);
            *(uint4 *)(sV + r * (DVV + 8) + 8 * ch) = x;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int item = tid + 256 * i;          // 128 dims x 8 column chunks
        const int d = item >> 3, cc = item & 7;  // cc: columns 8cc..8cc+7 of the tile
        if (t0 + 8 * cc >= p.T_pad) continue;
        bf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tok = vperm16(8 * cc + e);
            w[e] = __builtin_bit_cast(__bf16, sV[tok * (DVV + 8) + d]);
        }
        st16(p.vt + ((size_t)kvh * DVV + d) * p.T_pad + t0 + 8 * cc, w);
    }
}

}  // namespace

size_t prep_bytes(int T, int hkv)
{
    const size_t tp = (size_t)prep_tpad(T);
    const size_t kr = (tp * hkv * DQK * 2 + 255) & ~(size_t)255;
    const size_t vt = (tp * hkv * DVV * 2 + 255) & ~(size_t)255;
    return kr + vt;
}

void prep_carve(void *ws, int T, int hkv, KVPrep *p)
{
    p->T_pad = prep_tpad(T);
    p->k_rot = nullptr;
    p->kr = (uint16_t *)ws;
    const size_t kr = ((size_t)p->T_pad * hkv * DQK * 2 + 255) & ~(size_t)255;
    p->vt = (uint16_t *)((char *)ws + kr);
}

hipError_t launch_kv_prep_cached(const LayerArgs &a, const KVPrep &p, const CacheArgs &c, hipStream_t stream)
{
    const unsigned grid = (unsigned)((p.T_pad + PT - 1) / PT) * (unsigned)a.hkv;
    trace_begin(a.window >= 0 ? "kv_prep_cached_swa" : "kv_prep_cached_global", stream);
    kv_prep_cached_kernel<<<grid, 256, 0, stream>>>(a, p, c);
    trace_end(stream);
    return hipGetLastError();
}

hipError_t launch_kv_prep(const LayerArgs &a, const KVPrep &p, hipStream_t stream)
{
    const unsigned grid = (unsigned)((p.T_pad + PT - 1) / PT) * (unsigned)a.hkv;
    trace_begin(a.window >= 0 ? "kv_prep_swa" : "kv_prep_global", stream);
    kv_prep_kernel<<<grid, 256, 0, stream>>>(a, p);
    trace_end(stream);
    return hipGetLastError();
}

}  // namespace mimo
