// attn_fwd.hip -- prefill / training forward of the MiMo-V2.6-Flash attention layer on gfx950.
//
// Computes, per query row (token i, head h): RoPE on dims 0..63 of q and k (rotate-half, angle
// p * base^(-d/32)), scores q'.k'/sqrt(192) over the keys of the same sequence that the row may see
// (causal, and at most `window` keys back when window >= 0), a softmax whose denominator also holds
// exp(sink[h]), and out = softmax . (0.707 v).  Sources: miles docs "MiMo-V2.6-Flash" section 1 (hybrid
// attention, partial RoPE, V scale, RoPE bases) and section 5.4 (query + 128 previous keys); miles PR
// "feat(models): add MiMo-V2.6-Flash-RL support" (asymmetric Q/K vs V channels, sink on SWA layers).
//
// Design (gfx950, wave64):
//   * A workgroup of 4 waves owns 128 query rows: TT = 128 / GP consecutive tokens x GP query heads that
//     share one KV head.  Packing heads keeps a sliding-window tile's key span short (16 tokens + 128 keys
//     back) and lets all GP heads reuse each K/V tile staged in LDS.
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: the query is the MFMA column, so each lane owns one query
//     (lanes l and l ^ 32 split its keys); row max and row sum need one permlane32 swap, and the rescale of
//     the output accumulator is per lane.  O^T = V^T . P^T reuses the score registers as the B operand.
//   * K tiles are rotated while being staged into LDS (cos/sin from a table built in fp64); Q is rotated
//     once in registers.  V is staged transposed, with its 4-key chunks permuted so that the keys a lane
//     needs for P^T come out of LDS as one 16-byte read.
//   * Online softmax in base 2 (scale folded into one multiply); the sink starts the running max and sum.
//     Only tiles that cross the causal or window boundary evaluate the mask.  Key tiles outside the
//     window are never visited.
#include "device_common.hpp"
#include "internal.hpp"

namespace mimo {
namespace {

constexpr int BM = 128;        // query rows per workgroup
constexpr int BN = 64;         // keys per tile
constexpr int KS = DQK + 8;    // LDS row stride of the K tile (elements)
constexpr int VS = BN + 8;     // LDS row stride of the V^T tile (elements)

// LDS column chunk of a 4-key chunk inside a 16-key group: swaps the two chunk bits so that lane half hh
// reads keys {4hh..4hh+3, 8+4hh..8+4hh+3} as 8 consecutive elements.
__device__ __forceinline__ int vcol(int key4)
{
    int c4 = (key4 >> 2) & 3;
    return (key4 & ~15) | ((((c4 & 1) << 1) | (c4 >> 1)) << 2);
}

template <int GP, bool SINK, bool WIN>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const FwdArgs A)
{
    const LayerArgs &a = A.L;
    __shared__ __attribute__((aligned(16))) u16 sK[BN * KS];
    __shared__ __attribute__((aligned(16))) u16 sV[DVV * VS];

    constexpr int TT = BM / GP;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, c = lane & 31;
    const int G = a.hq / a.hkv;
    const int n_hg = G / GP;

    // ---- work item: KV head fastest (consecutive workgroups land on different XCDs and each XCD keeps
    // the K/V of "its" heads in L2), then head group, then token tile in reverse (longest causal work first).
    const int x = blockIdx.x;
    const int kvh = x % a.hkv;
    const int rest = x / a.hkv;
    const int hgi = rest % n_hg;
    const int tile = rest / n_hg;
    int ntiles = 0;
    for (int b = 0; b < a.batch; ++b) ntiles += (a.cu[b + 1] - a.cu[b] + TT - 1) / TT;
    if (tile >= ntiles) return;
    int tr = ntiles - 1 - tile;
    int seq_start = 0, seq_end = 0;
    for (int b = 0; b < a.batch; ++b) {
        seq_start = a.cu[b];
        seq_end = a.cu[b + 1];
        const int nt = (seq_end - seq_start + TT - 1) / TT;
        if (tr < nt) break;
        tr -= nt;
    }
    const int t0 = seq_start + tr * TT;
    const int t_last = min(t0 + TT - 1, seq_end - 1);
    const int h0 = kvh * G + hgi * GP;

    // ---- this lane's query row
    const int r = wave * 32 + c;
    const int qt = t0 + r / GP;
    const int qh = h0 + r % GP;
    const bool qvalid = qt < seq_end;
    const int qtl = qvalid ? qt : t_last;

    bf16x8 qf[12];
    {
        const u16 *qp = a.q + ((size_t)qtl * a.hq + qh) * DQK + 8 * hh;
#pragma unroll
        for (int s = 0; s < 12; ++s) qf[s] = ld16(qp + 16 * s);
        const float2 *cs = a.rope + (size_t)min(qtl - seq_start, a.rope_len - 1) * NHALF + 8 * hh;
        float2 c0[8], c1[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            c0[t] = cs[t];
            c1[t] = cs[16 + t];
        }
        rope_pair(qf[0], qf[2], c0);
        rope_pair(qf[1], qf[3], c1);
    }

    // ---- key range of the tile
    const int klo = WIN ? max(seq_start, t0 - a.window) : seq_start;
    const int khi = t_last;
    const int nkt = (khi - klo + BN) / BN;

    float m_run = -INFINITY, l_run = 0.f;
    if (SINK) {
        const float sk = a.sink[qh];
        if (sk > -INFINITY) {
            m_run = sk * LOG2E;
            l_run = hh == 0 ? 1.f : 0.f;
        }
    }
    f32x16 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x16{};

    // ---- staging registers (next tile prefetched while the current one is computed)
    uint4 kreg[6], vreg[4];
    float2 kcs[8];
    const int kk = tid >> 2, cg = tid & 3;       // K staging: key kk, chunks cg, cg+4 (rotated), 8+cg+4i
    const int vdc = tid & 15, vkc = tid >> 4;    // V staging: dims 8vdc..+7, keys 4vkc..+3

    auto load_tile = [&](int k0) {
        const int key = min(k0 + kk, khi);
        const u16 *kp = a.k + ((size_t)key * a.hkv + kvh) * DQK;
        kreg[0] = ldu4(kp + 8 * cg);
        kreg[1] = ldu4(kp + 8 * (cg + 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) kreg[2 + i] = ldu4(kp + 8 * (8 + cg + 4 * i));
        const float2 *cs = a.rope + (size_t)min(key - seq_start, a.rope_len - 1) * NHALF + 8 * cg;
#pragma unroll
        for (int t = 0; t < 8; ++t) kcs[t] = cs[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int vkey = min(k0 + 4 * vkc + i, khi);
            vreg[i] = ldu4(a.v + ((size_t)vkey * a.hkv + kvh) * DVV + 8 * vdc);
        }
    };
    auto store_tile = [&]() {
        bf16x8 x0 = __builtin_bit_cast(bf16x8, kreg[0]);
        bf16x8 x1 = __builtin_bit_cast(bf16x8, kreg[1]);
        rope_pair(x0, x1, kcs);
        u16 *kd = sK + kk * KS;
        st16(kd + 8 * cg, x0);
        st16(kd + 8 * (cg + 4), x1);
#pragma unroll
        for (int i = 0; i < 4; ++i) st16u(kd + 8 * (8 + cg + 4 * i), kreg[2 + i]);
        const int col = vcol(4 * vkc);
        const u16 *v0 = (const u16 *)&vreg[0], *v1 = (const u16 *)&vreg[1];
        const u16 *v2 = (const u16 *)&vreg[2], *v3 = (const u16 *)&vreg[3];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint2 w;
            w.x = (uint32_t)v0[e] | ((uint32_t)v1[e] << 16);
            w.y = (uint32_t)v2[e] | ((uint32_t)v3[e] << 16);
            *(uint2 *)(sV + (8 * vdc + e) * VS + col) = w;
        }
    };

    load_tile(klo);
    for (int it = 0; it < nkt; ++it) {
        const int k0 = klo + it * BN;
        __syncthreads();
        store_tile();
        __syncthreads();
        if (it + 1 < nkt) load_tile(k0 + BN);

        // S^T = K Q^T: two 32-key blocks x 12 k-steps of 16 dims
        f32x16 sacc[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            sacc[b] = f32x16{};
            const u16 *kr = sK + (32 * b + c) * KS + 8 * hh;
#pragma unroll
            for (int s = 0; s < 12; ++s) sacc[b] = mfma32(ld16(kr + 16 * s), qf[s], sacc[b]);
        }

        // mask (only on tiles that cross a boundary), online softmax in base 2
        const bool need_mask = (k0 + BN - 1 > t0) || (WIN && k0 < t_last - a.window);
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float s = sacc[b][j] * a.scale_log2;
                if (need_mask) {
                    const int key = k0 + 32 * b + 8 * (j >> 2) + 4 * hh + (j & 3);
                    const bool ok = key <= qt && (!WIN || key >= qt - a.window);
                    s = ok ? s : -INFINITY;
                }
                sacc[b][j] = s;
                mx = fmaxf(mx, s);
            }
        }
        mx = pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float psum = 0.f;
        bf16x8 pf[4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float p = fast_exp2(sacc[b][j] - m_use);
                psum += p;
                pf[2 * b + (j >> 3)][j & 7] = f2bf(p);
            }
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= alpha;

        // O^T += V^T P^T: four 32-dim blocks x four 16-key steps
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u16 *vr = sV + (32 * i + c) * VS + 8 * hh;
#pragma unroll
            for (int s = 0; s < 4; ++s) o[i] = mfma32(ld16(vr + 16 * s), pf[s], o[i]);
        }
    }

    // ---- epilogue: out = 0.707 * O / l, LSE = ln(l) + max
    const float l_tot = pair_sum(l_run);
    if (qvalid) {
        const float inv = VSCALE / l_tot;
        u16 *op = A.out + ((size_t)qt * a.hq + qh) * DVV + 4 * hh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = f2bf(o[i][4 * jj + t] * inv);
                *(uint2 *)(op + 32 * i + 8 * jj) = __builtin_bit_cast(uint2, w);
            }
        }
        if (A.lse && hh == 0) A.lse[(size_t)qh * a.T + qt] = (m_run + __log2f(l_tot)) * LN2;
    }
}

template <int GP>
hipError_t launch_gp(const FwdArgs &A, hipStream_t stream)
{
    const LayerArgs &a = A.L;
    constexpr int TT = BM / GP;
    const int G = a.hq / a.hkv;
    // upper bound on the number of token tiles: sum ceil(len/TT) <= ceil(T/TT) + batch
    const long tiles = (long)(a.T + TT - 1) / TT + a.batch;
    const long grid = tiles * (G / GP) * a.hkv;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    const bool sink = a.sink != nullptr, win = a.window >= 0;
    trace_begin(win ? "attn_fwd_swa" : "attn_fwd_global", stream);
    if (sink && win) attn_fwd_kernel<GP, true, true><<<(unsigned)grid, 256, 0, stream>>>(A);
    else if (sink) attn_fwd_kernel<GP, true, false><<<(unsigned)grid, 256, 0, stream>>>(A);
    else if (win) attn_fwd_kernel<GP, false, true><<<(unsigned)grid, 256, 0, stream>>>(A);
    else attn_fwd_kernel<GP, false, false><<<(unsigned)grid, 256, 0, stream>>>(A);
    trace_end(stream);
    return hipGetLastError();
}

__global__ void rope_table_kernel(float2 *t, int npos, double base)
{
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)npos * NHALF) return;
    const int pos = (int)(idx / NHALF), d = (int)(idx % NHALF);
    const double ang = (double)pos * pow(base, -(double)d / (double)NHALF);
    double s, c;
    sincos(ang, &s, &c);
    t[idx] = make_float2((float)c, (float)s);
}

}  // namespace

bool fwd_group_supported(int group) { return group >= 1; }

hipError_t launch_fwd(const FwdArgs &A, hipStream_t stream)
{
    const LayerArgs &a = A.L;
    const int G = a.hq / a.hkv;
    // pack up to 8 heads of a group: 16 tokens x 8 heads per workgroup for sliding-window layers (short key
    // span), and the same for causal layers (each K/V tile serves 8 heads; little waste on the diagonal).
    if (G % 8 == 0) return launch_gp<8>(A, stream);
    if (G % 4 == 0) return launch_gp<4>(A, stream);
    if (G % 2 == 0) return launch_gp<2>(A, stream);
    return launch_gp<1>(A, stream);
}

hipError_t launch_rope_table(float2 *table, int npos, double base, hipStream_t stream)
{
    const long n = (long)npos * NHALF;
    const long blocks = (n + 255) / 256;
    rope_table_kernel<<<(unsigned)blocks, 256, 0, stream>>>(table, npos, base);
    return hipGetLastError();
}

}  // namespace mimo
