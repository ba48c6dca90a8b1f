// attn_decode.hip -- one decode step of the MiMo-V2.6-Flash attention layer against a KV cache (gfx950).
//
// For sequence b with its new token at position p: q' = RoPE(q, p), k_new' = RoPE(k_new, p); the cache
// rows of b hold keys already rotated at their own positions and unscaled values.  The query attends the
// last min(n_b, window) cache rows (all of them for window = -1) plus the new token, with the per-head sink
// in the softmax denominator, and out = 0.707 * softmax . v.  Sources: miles PR "feat(models): add
// MiMo-V2.6-Flash-RL support" (rollout engine window = query + 128 previous keys); miles docs
// "MiMo-V2.6-Flash" section 1 (sink, V scale, RoPE) and section 3.2 (sliding-window KV pools).
//
// Design: the step is HBM-bound (640 bytes of cache per key and KV head against 16 x 640 flops), so the
// kernel streams each cache row exactly once.  A one-wave workgroup owns (sequence, KV head, split of
// up to split_len rows) and walks it in 32-row chunks: K goes straight from HBM into MFMA A operands
// (S^T = K q^T with the G query heads of the group as MFMA columns), V is staged transposed through LDS
// for O^T = V^T P^T.  The next chunk is loaded while the current one is computed.  Each split writes an
// unnormalised partial (o, running max, running sum); the combine kernel merges the splits with the sink
// and the new token (whose rotation is computed there in double precision).
#include "device_common.hpp"
#include "internal.hpp"

namespace mimo {
namespace {

constexpr int CH = 32;            // cache rows per chunk
constexpr int VTS = CH + 8;       // LDS stride of the V^T chunk

__device__ __forceinline__ int vcol(int key4)
{
    const int c4 = (key4 >> 2) & 3;
    return (key4 & ~15) | ((((c4 & 1) << 1) | (c4 >> 1)) << 2);
}

__device__ __forceinline__ double inv_freq(double base, int d) { return pow(base, -(double)d / (double)NHALF); }

__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeArgs A)
{
    __shared__ __attribute__((aligned(16))) u16 sVT[DVV * VTS];
    const int lane = threadIdx.x, hh = lane >> 5, c = lane & 31;
    const int G = A.hq / A.hkv;
    const int ngrp = (G + 31) / 32;          // the group's query heads in blocks of 32 MFMA columns
    int w = blockIdx.x;
    const int split = w % A.splits;
    w /= A.splits;
    const int hgrp = w % ngrp;
    w /= ngrp;
    const int kvh = w % A.hkv;
    const int b = w / A.hkv;
    if (b >= A.batch) return;

    int c0 = A.cu_cache[b];
    const int c1 = A.cu_cache[b + 1];
    if (A.window >= 0 && c1 - c0 > A.window) c0 = c1 - A.window;
    const int n = c1 - c0;
    const int ks = split * A.split_len;
    const int ke = min(n, ks + A.split_len);
    const int gi = hgrp * 32 + c;            // this lane's head inside the group
    const bool hvalid = gi < G;
    const int h = kvh * G + (hvalid ? gi : G - 1);   // spare MFMA columns repeat the group's last head
    const size_t part = ((size_t)b * A.hq + h) * A.splits + split;

    if (ks >= ke) {                          // nothing cached in this split: an empty partial
        if (hvalid) {
            if (hh == 0) {
                A.part_ml[part * 2 + 0] = -INFINITY;
                A.part_ml[part * 2 + 1] = 0.f;
            }
            float *po = A.part_o + part * DVV;
            for (int d = hh; d < DVV; d += 2) po[d] = 0.f;
        }
        return;
    }

    // rotated query (bf16) as the B operand: column = head, dims 16s + 8hh + t
    bf16x8 qf[12];
    {
        const u16 *qp = A.q + ((size_t)b * A.hq + h) * DQK + 8 * hh;
#pragma unroll
        for (int s = 0; s < 12; ++s) qf[s] = ld16(qp + 16 * s);
        const double pos = (double)A.positions[b];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float2 cs[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                double sn, cn;
                sincos(pos * inv_freq(A.rope_base, 16 * s + 8 * hh + t), &sn, &cn);
                cs[t] = make_float2((float)cn, (float)sn);
            }
            rope_pair(qf[s], qf[s + 2], cs);
        }
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x16{};

    const u16 *kbase = A.k_cache + (size_t)kvh * DQK + 8 * hh;
    const u16 *vbase = A.v_cache + (size_t)kvh * DVV;
    const size_t krow = (size_t)A.hkv * DQK, vrow = (size_t)A.hkv * DVV;
    const int vdc = lane & 15, vk4 = lane >> 4;   // V staging: dims 8vdc..+7, keys 4vk4..+3 (+16 second pass)

    uint4 kreg[12], vreg[8];
    auto load_chunk = [&](int k) {
        const size_t row = (size_t)c0 + min(k + c, ke - 1);
#pragma unroll
        for (int s = 0; s < 12; ++s) kreg[s] = ldu4(kbase + row * krow + 16 * s);
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t vr = (size_t)c0 + min(k + 16 * p + 4 * vk4 + i, ke - 1);
                vreg[4 * p + i] = ldu4(vbase + vr * vrow + 8 * vdc);
            }
    };

    load_chunk(ks);
    for (int k = ks; k < ke; k += CH) {
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int col = vcol(16 * p + 4 * vk4);
            const u16 *v0 = (const u16 *)&vreg[4 * p + 0], *v1 = (const u16 *)&vreg[4 * p + 1];
            const u16 *v2 = (const u16 *)&vreg[4 * p + 2], *v3 = (const u16 *)&vreg[4 * p + 3];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint2 wv;
                wv.x = (uint32_t)v0[e] | ((uint32_t)v1[e] << 16);
                wv.y = (uint32_t)v2[e] | ((uint32_t)v3[e] << 16);
                *(uint2 *)(sVT + (8 * vdc + e) * VTS + col) = wv;
            }
        }
        f32x16 sacc = f32x16{};
#pragma unroll
        for (int s = 0; s < 12; ++s) sacc = mfma32(__builtin_bit_cast(bf16x8, kreg[s]), qf[s], sacc);
        __syncthreads();
        if (k + CH < ke) load_chunk(k + CH);

        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int key = k + 8 * (j >> 2) + 4 * hh + (j & 3);
            const float s = key < ke ? sacc[j] * A.scale_log2 : -INFINITY;
            sacc[j] = s;
            mx = fmaxf(mx, s);
        }
        mx = pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        float psum = 0.f;
        bf16x8 pf[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = fast_exp2(sacc[j] - m_new);
            psum += p;
            pf[j >> 3][j & 7] = f2bf(p);
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[i] *= alpha;
            const u16 *vr = sVT + (32 * i + c) * VTS + 8 * hh;
#pragma unroll
            for (int s = 0; s < 2; ++s) o[i] = mfma32(ld16(vr + 16 * s), pf[s], o[i]);
        }
    }

    const float l_tot = pair_sum(l_run);
    if (hvalid) {
        if (hh == 0) {
            A.part_ml[part * 2 + 0] = m_run;
            A.part_ml[part * 2 + 1] = l_tot;
        }
        float *po = A.part_o + part * DVV + 4 * hh;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *(float4 *)(po + 32 * i + 8 * jj) =
                    make_float4(o[i][4 * jj], o[i][4 * jj + 1], o[i][4 * jj + 2], o[i][4 * jj + 3]);
    }
}

// One wave per (sequence, query head): merge the splits, the new token and the sink.
__global__ __launch_bounds__(64) void decode_combine_kernel(const DecodeArgs A)
{
    const int lane = threadIdx.x;
    const int b = blockIdx.x / A.hq, h = blockIdx.x % A.hq;
    const int G = A.hq / A.hkv, kvh = h / G;
    const double pos = (double)A.positions[b];

    // score of the new token: rotate q and k_new (dims 3*lane .. 3*lane+2 of 192) in fp32 from fp64 angles
    const u16 *qp = A.q + ((size_t)b * A.hq + h) * DQK;
    const u16 *kp = A.k_new + ((size_t)b * A.hkv + kvh) * DQK;
    float dot = 0.f;
    if (lane < NHALF) {
        double sn, cn;
        sincos(pos * inv_freq(A.rope_base, lane), &sn, &cn);
        const float cf = (float)cn, sf = (float)sn;
        const float q0 = bf2f(__builtin_bit_cast(__bf16, qp[lane])), q1 = bf2f(__builtin_bit_cast(__bf16, qp[lane + 32]));
        const float k0 = bf2f(__builtin_bit_cast(__bf16, kp[lane])), k1 = bf2f(__builtin_bit_cast(__bf16, kp[lane + 32]));
        const float qa = q0 * cf - q1 * sf, qb = q1 * cf + q0 * sf;
        const float ka = k0 * cf - k1 * sf, kb = k1 * cf + k0 * sf;
        dot = qa * ka + qb * kb;
    }
    for (int d = 64 + lane; d < DQK; d += 64)
        dot += bf2f(__builtin_bit_cast(__bf16, qp[d])) * bf2f(__builtin_bit_cast(__bf16, kp[d]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
    const float s_new = dot * A.scale_log2;

    const float *ml = A.part_ml + ((size_t)b * A.hq + h) * A.splits * 2;
    const float *po = A.part_o + ((size_t)b * A.hq + h) * A.splits * DVV;
    float M = s_new;
    const float sk = A.sink ? A.sink[h] * LOG2E : -INFINITY;
    M = fmaxf(M, sk);
    for (int s = 0; s < A.splits; ++s) M = fmaxf(M, ml[2 * s]);
    const float w_new = fast_exp2(s_new - M);
    float L = w_new + (sk > -INFINITY ? fast_exp2(sk - M) : 0.f);
    const u16 *vp = A.v_new + ((size_t)b * A.hkv + kvh) * DVV;
    float o0 = w_new * bf2f(__builtin_bit_cast(__bf16, vp[2 * lane]));
    float o1 = w_new * bf2f(__builtin_bit_cast(__bf16, vp[2 * lane + 1]));
    for (int s = 0; s < A.splits; ++s) {
        const float m = ml[2 * s];
        if (m == -INFINITY) continue;
        const float wgt = fast_exp2(m - M);
        L += wgt * ml[2 * s + 1];
        o0 += wgt * po[(size_t)s * DVV + 2 * lane];
        o1 += wgt * po[(size_t)s * DVV + 2 * lane + 1];
    }
    const float inv = VSCALE / L;
    u16 *out = A.out + ((size_t)b * A.hq + h) * DVV + 2 * lane;
    out[0] = __builtin_bit_cast(u16, f2bf(o0 * inv));
    out[1] = __builtin_bit_cast(u16, f2bf(o1 * inv));
}

}  // namespace

bool decode_group_supported(int group) { return group >= 1; }

void decode_split_plan(int batch, int max_cache_len, int hq, int hkv, int window, int *splits, int *split_len)
{
    (void)batch;
    (void)hq;
    (void)hkv;
    int n = max_cache_len;
    if (window >= 0 && window < n) n = window;
    // at most 32 splits, each a multiple of the chunk and at least 1024 rows
    int len = (n + 31) / 32;
    len = (len + CH - 1) / CH * CH;
    if (len < 1024) len = 1024;
    int s = (n + len - 1) / len;
    if (s < 1) s = 1;
    *splits = s;
    *split_len = len;
}

size_t decode_workspace_bytes(int batch, int max_cache_len, int hq, int window)
{
    int splits, len;
    decode_split_plan(batch, max_cache_len, hq, 1, window, &splits, &len);
    const size_t po = ((size_t)batch * hq * splits * DVV * sizeof(float) + 255) & ~(size_t)255;
    const size_t ml = (size_t)batch * hq * splits * 2 * sizeof(float);
    return po + ml;
}

hipError_t launch_decode(const DecodeArgs &A, hipStream_t stream)
{
    const int G = A.hq / A.hkv;
    const long waves = (long)A.batch * A.hkv * ((G + 31) / 32) * A.splits;
    if (waves > 0x7fffffffL || (long)A.batch * A.hq > 0x7fffffffL) return hipErrorInvalidConfiguration;
    trace_begin(A.window >= 0 ? "decode_split_swa" : "decode_split_global", stream);
    decode_split_kernel<<<(unsigned)waves, 64, 0, stream>>>(A);
    trace_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    trace_begin("decode_combine", stream);
    decode_combine_kernel<<<(unsigned)(A.batch * A.hq), 64, 0, stream>>>(A);
    trace_end(stream);
    return hipGetLastError();
}

}  // namespace mimo
