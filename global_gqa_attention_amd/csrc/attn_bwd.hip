// attn_bwd.hip -- training backward of the MiMo-V2.6-Flash attention layer on gfx950.
//
// The exact gradient of the forward in attn_fwd.hip, with the forward outputs given (O, LSE):
//   D_i = dO_i . O_i,  P_ij = exp(s_ij - LSE_i),  dP_ij = 0.707 dO_i . v_j,  dS_ij = P_ij (dP_ij - D_i)
//   dv_j = 0.707 sum_i P_ij dO_i        (summed over the query heads of the KV group)
//   dk_j = R_j^T sum_i dS_ij q'_i / sqrt(192),  dq_i = R_i^T sum_j dS_ij k'_j / sqrt(192)
//   dsink_h = -sum_i exp(sink_h - LSE_i) D_i
// where R is the RoPE rotation at the row's position (its transpose rotates by the opposite angle).
// Sources: miles docs "MiMo-V2.6-Flash" sections 1 and 5.4 (the trainer's fused attention carries the
// sink and the V scale through training); miles PR "feat(models): add MiMo-V2.6-Flash-RL support".
//
// Kernels, all on the caller's stream, no atomics (every output is written by exactly one workgroup and
// dsink is summed in a fixed order, so results are bitwise repeatable):
//   1. bwd_pre:   D for every (token, head) row.
//   2. bwd_dsink: one workgroup per head, fixed-order tree sum (only when a sink is given).
//   3. bwd_dkdv:  key-major.  A workgroup owns 128 keys of one KV head (32 per wave, the key is the MFMA
//                 column so each lane owns one key) and walks every (query head of the group, 64-query
//                 tile) that sees them: S = Q K^T, P, dP = dO V^T, dS, then dV^T += dO^T P and
//                 dK^T += Q^T dS with K/V resident in registers and Q/dO staged in LDS in both layouts.
//   4. bwd_dq:    query-major, laid out like the forward: S^T = K Q^T, P^T, dP^T = V dO^T, dS^T, then
//                 dQ^T += K^T dS^T with K staged in LDS row-major and transposed.
// RoPE is applied when Q/K are loaded and undone (transposed rotation) in the dq/dk epilogues.
#include "device_common.hpp"
#include "internal.hpp"

namespace mimo {
namespace {

constexpr float RSQRT_DQK = 0.07216878364870322f;   // 1 / sqrt(192)

__device__ __forceinline__ int vcol(int r4)
{
    const int c4 = (r4 >> 2) & 3;
    return (r4 & ~15) | ((((c4 & 1) << 1) | (c4 >> 1)) << 2);
}

// Copy a row-major R x C bf16 tile into its transpose (C rows of R), with the 4-row chunks of every 16-row
// group permuted as vcol() says, so that an MFMA A-operand read of 8 consecutive elements returns the rows
// in the order the score registers hold them.
template <int R, int C, int SS, int DS>
__device__ __forceinline__ void transpose_tile(const u16 *src, u16 *dst, int tid)
{
    constexpr int NB = (R / 4) * (C / 8);
    for (int blk = tid; blk < NB; blk += 256) {
        const int r4 = blk % (R / 4), c8 = blk / (R / 4);
        uint4 x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = *(const uint4 *)(src + (4 * r4 + i) * SS + 8 * c8);
        const u16 *p0 = (const u16 *)&x[0], *p1 = (const u16 *)&x[1];
        const u16 *p2 = (const u16 *)&x[2], *p3 = (const u16 *)&x[3];
        const int col = vcol(4 * r4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint2 w;
            w.x = (uint32_t)p0[e] | ((uint32_t)p1[e] << 16);
            w.y = (uint32_t)p2[e] | ((uint32_t)p3[e] << 16);
            *(uint2 *)(dst + (8 * c8 + e) * DS + col) = w;
        }
    }
}

// Transposed RoPE of a 32-dim block pair held in C layout: x0 = dims 8(j/4)+4hh+j%4, x1 the same dims + 32.
__device__ __forceinline__ void rope_back(f32x16 &x0, f32x16 &x1, const float2 *cs, int hh)
{
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float2 e = cs[8 * (j >> 2) + 4 * hh + (j & 3)];
        const float a = x0[j], b = x1[j];
        x0[j] = a * e.x + b * e.y;
        x1[j] = b * e.x - a * e.y;
    }
}

// ------------------------------------------------------------------------------------------------------
// 1. D = rowsum(dO * O)
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdArgs A)
{
    const int tid = threadIdx.x, g = tid >> 4, sub = tid & 15;
    const long rows = (long)A.L.T * A.L.hq;
    const long r0 = (long)blockIdx.x * 64;
    for (long r = r0 + g; r < rows && r < r0 + 64; r += 16) {
        const bf16x8 a = ld16(A.dout + r * DVV + 8 * sub);
        const bf16x8 b = ld16(A.out + r * DVV + 8 * sub);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s += bf2f(a[e]) * bf2f(b[e]);
        s += __shfl_xor(s, 8, 16);
        s += __shfl_xor(s, 4, 16);
        s += __shfl_xor(s, 2, 16);
        s += __shfl_xor(s, 1, 16);
        if (sub == 0) {
            const int t = (int)(r / A.L.hq), h = (int)(r % A.L.hq);
            A.delta[(size_t)h * A.L.T + t] = s;
        }
    }
}

// ------------------------------------------------------------------------------------------------------
// 2. dsink_h = -sum_t exp(sink_h - LSE_t) D_t, fixed order
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dsink_kernel(const BwdArgs A)
{
    __shared__ float red[256];
    const int h = blockIdx.x, tid = threadIdx.x;
    const float sk = A.L.sink[h];
    float acc = 0.f;
    if (sk > -INFINITY) {
        const float *lse = A.lse + (size_t)h * A.L.T, *dl = A.delta + (size_t)h * A.L.T;
        for (int t = tid; t < A.L.T; t += 256) acc -= expf(sk - lse[t]) * dl[t];
    }
    red[tid] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
    }
    if (tid == 0) A.dsink[h] = red[0];
}

__global__ void zero_kernel(float *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// ------------------------------------------------------------------------------------------------------
// 3. dK, dV (key-major)
// ------------------------------------------------------------------------------------------------------
constexpr int NKB = 128;        // keys per workgroup (32 per wave)
constexpr int MQ = 64;          // queries per step
constexpr int QS = DQK + 8;     // row-major Q stride
constexpr int OS = DVV + 8;     // row-major dO stride
constexpr int TS = MQ + 8;      // transposed tiles: stride over queries

template <bool WIN>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(const BwdArgs A)
{
    const LayerArgs &a = A.L;
    __shared__ __attribute__((aligned(16))) u16 sQ[MQ * QS];
    __shared__ __attribute__((aligned(16))) u16 sQT[DQK * TS];
    __shared__ __attribute__((aligned(16))) u16 sO[MQ * OS];
    __shared__ __attribute__((aligned(16))) u16 sOT[DVV * TS];
    __shared__ __attribute__((aligned(16))) float sL[MQ];
    __shared__ __attribute__((aligned(16))) float sD[MQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, c = lane & 31;
    const int G = a.hq / a.hkv;

    // ---- work item: KV head fastest; key tiles of the sequences from last to first
    const int x = blockIdx.x;
    const int kvh = x % a.hkv;
    int tile = x / a.hkv;
    int seq_start = 0, seq_end = 0;
    bool found = false;
    for (int b = a.batch - 1; b >= 0; --b) {
        seq_start = a.cu[b];
        seq_end = a.cu[b + 1];
        const int nt = (seq_end - seq_start + NKB - 1) / NKB;
        if (tile < nt) {
            found = true;
            break;
        }
        tile -= nt;
    }
    if (!found) return;
    const int kb0 = seq_start + tile * NKB;
    const int kb_last = min(kb0 + NKB - 1, seq_end - 1);

    // ---- this lane's key, K (rotated) and V as B operands
    const int kw0 = kb0 + 32 * wave;
    const int kj = kw0 + c;
    const bool kvalid = kj <= kb_last;
    const int kjl = kvalid ? kj : kb_last;
    bf16x8 kf[12], vf[8];
    {
        const u16 *kp = a.k + ((size_t)kjl * a.hkv + kvh) * DQK + 8 * hh;
#pragma unroll
        for (int s = 0; s < 12; ++s) kf[s] = ld16(kp + 16 * s);
        const u16 *vp = a.v + ((size_t)kjl * a.hkv + kvh) * DVV + 8 * hh;
#pragma unroll
        for (int s = 0; s < 8; ++s) vf[s] = ld16(vp + 16 * s);
        const float2 *cs = a.rope + (size_t)min(kjl - seq_start, a.rope_len - 1) * NHALF + 8 * hh;
        float2 c0[8], c1[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            c0[t] = cs[t];
            c1[t] = cs[16 + t];
        }
        rope_pair(kf[0], kf[2], c0);
        rope_pair(kf[1], kf[3], c1);
    }

    f32x16 dk[6], dv[4];
#pragma unroll
    for (int i = 0; i < 6; ++i) dk[i] = f32x16{};
#pragma unroll
    for (int i = 0; i < 4; ++i) dv[i] = f32x16{};

    const int q_lo = kb0;
    const int q_hi = WIN ? min(seq_end - 1, kb_last + a.window) : seq_end - 1;
    const int nq = (q_hi - q_lo + MQ) / MQ;
    const int nsteps = nq * G;

    // ---- staging: Q row (rotated) + dO row + LSE/D for step (h, q0)
    uint4 qreg[6], oreg[4];
    float2 qcs[8];
    float ld_val = 0.f;
    const int sr = tid >> 2, cg = tid & 3;
    auto load_step = [&](int step) {
        const int h = kvh * G + step / nq;
        const int q0 = q_lo + (step % nq) * MQ;
        const int qi = min(q0 + sr, q_hi);
        const u16 *qp = a.q + ((size_t)qi * a.hq + h) * DQK;
        qreg[0] = ldu4(qp + 8 * cg);
        qreg[1] = ldu4(qp + 8 * (cg + 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) qreg[2 + i] = ldu4(qp + 8 * (8 + cg + 4 * i));
        const float2 *cs = a.rope + (size_t)min(qi - seq_start, a.rope_len - 1) * NHALF + 8 * cg;
#pragma unroll
        for (int t = 0; t < 8; ++t) qcs[t] = cs[t];
        const u16 *op = A.dout + ((size_t)qi * a.hq + h) * DVV;
#pragma unroll
        for (int i = 0; i < 4; ++i) oreg[i] = ldu4(op + 8 * (cg + 4 * i));
        if (tid < MQ) ld_val = A.lse[(size_t)h * a.T + min(q0 + tid, q_hi)] * LOG2E;
        else if (tid < 2 * MQ) ld_val = A.delta[(size_t)h * a.T + min(q0 + tid - MQ, q_hi)];
    };
    auto store_step = [&]() {
        bf16x8 x0 = __builtin_bit_cast(bf16x8, qreg[0]);
        bf16x8 x1 = __builtin_bit_cast(bf16x8, qreg[1]);
        rope_pair(x0, x1, qcs);
        u16 *qd = sQ + sr * QS;
        st16(qd + 8 * cg, x0);
        st16(qd + 8 * (cg + 4), x1);
#pragma unroll
        for (int i = 0; i < 4; ++i) st16u(qd + 8 * (8 + cg + 4 * i), qreg[2 + i]);
        u16 *od = sO + sr * OS;
#pragma unroll
        for (int i = 0; i < 4; ++i) st16u(od + 8 * (cg + 4 * i), oreg[i]);
        if (tid < MQ) sL[tid] = ld_val;
        else if (tid < 2 * MQ) sD[tid - MQ] = ld_val;
    };

    if (nsteps > 0) load_step(0);
    for (int step = 0; step < nsteps; ++step) {
        const int q0 = q_lo + (step % nq) * MQ;
        __syncthreads();
        store_step();
        __syncthreads();
        transpose_tile<MQ, DQK, QS, TS>(sQ, sQT, tid);
        transpose_tile<MQ, DVV, OS, TS>(sO, sOT, tid);
        __syncthreads();
        if (step + 1 < nsteps) load_step(step + 1);

        // does any query of this step see any key of this wave?
        const bool active = (q0 + MQ - 1 >= kw0) && (kw0 <= kb_last) && (!WIN || q0 <= kw0 + 31 + a.window);
        if (!active) continue;
        const bool need_mask = (q0 < kw0 + 31) || (q0 + MQ - 1 > q_hi) ||
                               (WIN && q0 + MQ - 1 > kw0 + a.window) || (kw0 + 31 > kb_last);

        f32x16 sacc[2], dpacc[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            sacc[qb] = f32x16{};
            dpacc[qb] = f32x16{};
            const u16 *qr = sQ + (32 * qb + c) * QS + 8 * hh;
#pragma unroll
            for (int s = 0; s < 12; ++s) sacc[qb] = mfma32(ld16(qr + 16 * s), kf[s], sacc[qb]);
            const u16 *orow = sO + (32 * qb + c) * OS + 8 * hh;
#pragma unroll
            for (int s = 0; s < 8; ++s) dpacc[qb] = mfma32(ld16(orow + 16 * s), vf[s], dpacc[qb]);
        }
        bf16x8 pb[4], sb[4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int ql = 32 * qb + 8 * jj + 4 * hh;
                const float4 L4 = *(const float4 *)(sL + ql);
                const float4 D4 = *(const float4 *)(sD + ql);
                const float Lv[4] = {L4.x, L4.y, L4.z, L4.w};
                const float Dv[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int j = 4 * jj + t;
                    float p = fast_exp2(sacc[qb][j] * a.scale_log2 - Lv[t]);
                    if (need_mask) {
                        const int qi = q0 + ql + t;
                        const bool ok = kvalid && qi >= kj && qi <= q_hi && (!WIN || qi - kj <= a.window);
                        p = ok ? p : 0.f;
                    }
                    const float ds = p * (VSCALE * dpacc[qb][j] - Dv[t]);
                    pb[2 * qb + (j >> 3)][j & 7] = f2bf(p);
                    sb[2 * qb + (j >> 3)][j & 7] = f2bf(ds);
                }
            }
        }
        // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u16 *tr = sOT + (32 * i + c) * TS + 8 * hh;
#pragma unroll
            for (int s = 0; s < 4; ++s) dv[i] = mfma32(ld16(tr + 16 * s), pb[s], dv[i]);
        }
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const u16 *tr = sQT + (32 * i + c) * TS + 8 * hh;
#pragma unroll
            for (int s = 0; s < 4; ++s) dk[i] = mfma32(ld16(tr + 16 * s), sb[s], dk[i]);
        }
    }

    // ---- epilogue: dv = 0.707 * dV^T, dk = R^T dK^T / sqrt(192)
    if (kvalid) {
        u16 *dvp = A.dv + ((size_t)kj * a.hkv + kvh) * DVV + 4 * hh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = f2bf(dv[i][4 * jj + t] * VSCALE);
                *(uint2 *)(dvp + 32 * i + 8 * jj) = __builtin_bit_cast(uint2, w);
            }
        }
        const float2 *cs = a.rope + (size_t)min(kj - seq_start, a.rope_len - 1) * NHALF;
        rope_back(dk[0], dk[1], cs, hh);
        u16 *dkp = A.dk + ((size_t)kj * a.hkv + kvh) * DQK + 4 * hh;
#pragma unroll
        for (int i = 0; i < 6; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = f2bf(dk[i][4 * jj + t] * RSQRT_DQK);
                *(uint2 *)(dkp + 32 * i + 8 * jj) = __builtin_bit_cast(uint2, w);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------------
// 4. dQ (query-major)
// ------------------------------------------------------------------------------------------------------
constexpr int BM = 128;        // query rows per workgroup
constexpr int BN = 64;         // keys per tile
constexpr int KS = DQK + 8;
constexpr int VS = DVV + 8;
constexpr int KTS = BN + 8;

template <int GP, bool WIN>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(const BwdArgs A)
{
    const LayerArgs &a = A.L;
    __shared__ __attribute__((aligned(16))) u16 sK[BN * KS];
    __shared__ __attribute__((aligned(16))) u16 sKT[DQK * KTS];
    __shared__ __attribute__((aligned(16))) u16 sV[BN * VS];

    constexpr int TT = BM / GP;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, c = lane & 31;
    const int G = a.hq / a.hkv;
    const int n_hg = G / GP;

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

    const int r = wave * 32 + c;
    const int qt = t0 + r / GP;
    const int qh = h0 + r % GP;
    const bool qvalid = qt < seq_end;
    const int qtl = qvalid ? qt : t_last;

    bf16x8 qf[12], of[8];
    const float2 *qcs = a.rope + (size_t)min(qtl - seq_start, a.rope_len - 1) * NHALF;
    {
        const u16 *qp = a.q + ((size_t)qtl * a.hq + qh) * DQK + 8 * hh;
#pragma unroll
        for (int s = 0; s < 12; ++s) qf[s] = ld16(qp + 16 * s);
        const u16 *op = A.dout + ((size_t)qtl * a.hq + qh) * DVV + 8 * hh;
#pragma unroll
        for (int s = 0; s < 8; ++s) of[s] = ld16(op + 16 * s);
        float2 c0[8], c1[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            c0[t] = qcs[8 * hh + t];
            c1[t] = qcs[16 + 8 * hh + t];
        }
        rope_pair(qf[0], qf[2], c0);
        rope_pair(qf[1], qf[3], c1);
    }
    const float Lq = A.lse[(size_t)qh * a.T + qtl] * LOG2E;
    const float Dq = A.delta[(size_t)qh * a.T + qtl];

    const int klo = WIN ? max(seq_start, t0 - a.window) : seq_start;
    const int khi = t_last;
    const int nkt = (khi - klo + BN) / BN;

    f32x16 dq[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) dq[i] = f32x16{};

    uint4 kreg[6], vreg[4];
    float2 kcs[8];
    const int kk = tid >> 2, cg = tid & 3;
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
        const u16 *vp = a.v + ((size_t)key * a.hkv + kvh) * DVV;
#pragma unroll
        for (int i = 0; i < 4; ++i) vreg[i] = ldu4(vp + 8 * (cg + 4 * i));
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
        u16 *vd = sV + kk * VS;
#pragma unroll
        for (int i = 0; i < 4; ++i) st16u(vd + 8 * (cg + 4 * i), vreg[i]);
    };

    load_tile(klo);
    for (int it = 0; it < nkt; ++it) {
        const int k0 = klo + it * BN;
        __syncthreads();
        store_tile();
        __syncthreads();
        transpose_tile<BN, DQK, KS, KTS>(sK, sKT, tid);
        __syncthreads();
        if (it + 1 < nkt) load_tile(k0 + BN);

        const bool need_mask = (k0 + BN - 1 > t0) || (WIN && k0 < t_last - a.window);
        f32x16 sacc[2], dpacc[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            sacc[b] = f32x16{};
            dpacc[b] = f32x16{};
            const u16 *kr = sK + (32 * b + c) * KS + 8 * hh;
#pragma unroll
            for (int s = 0; s < 12; ++s) sacc[b] = mfma32(ld16(kr + 16 * s), qf[s], sacc[b]);
            const u16 *vr = sV + (32 * b + c) * VS + 8 * hh;
#pragma unroll
            for (int s = 0; s < 8; ++s) dpacc[b] = mfma32(ld16(vr + 16 * s), of[s], dpacc[b]);
        }
        bf16x8 sb[4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float p = fast_exp2(sacc[b][j] * a.scale_log2 - Lq);
                if (need_mask) {
                    const int key = k0 + 32 * b + 8 * (j >> 2) + 4 * hh + (j & 3);
                    const bool ok = key <= qt && key <= khi && (!WIN || key >= qt - a.window);
                    p = ok ? p : 0.f;
                }
                sb[2 * b + (j >> 3)][j & 7] = f2bf(p * (VSCALE * dpacc[b][j] - Dq));
            }
        }
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const u16 *tr = sKT + (32 * i + c) * KTS + 8 * hh;
#pragma unroll
            for (int s = 0; s < 4; ++s) dq[i] = mfma32(ld16(tr + 16 * s), sb[s], dq[i]);
        }
    }

    if (qvalid) {
        rope_back(dq[0], dq[1], qcs, hh);
        u16 *dqp = A.dq + ((size_t)qt * a.hq + qh) * DQK + 4 * hh;
#pragma unroll
        for (int i = 0; i < 6; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = f2bf(dq[i][4 * jj + t] * RSQRT_DQK);
                *(uint2 *)(dqp + 32 * i + 8 * jj) = __builtin_bit_cast(uint2, w);
            }
        }
    }
}

template <int GP>
hipError_t launch_dq(const BwdArgs &A, hipStream_t stream)
{
    const LayerArgs &a = A.L;
    constexpr int TT = BM / GP;
    const int G = a.hq / a.hkv;
    const long tiles = (long)(a.T + TT - 1) / TT + a.batch;
    const long grid = tiles * (G / GP) * a.hkv;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    trace_begin(a.window >= 0 ? "bwd_dq_swa" : "bwd_dq_global", stream);
    if (a.window >= 0) bwd_dq_kernel<GP, true><<<(unsigned)grid, 256, 0, stream>>>(A);
    else bwd_dq_kernel<GP, false><<<(unsigned)grid, 256, 0, stream>>>(A);
    trace_end(stream);
    return hipGetLastError();
}

}  // namespace

bool bwd_group_supported(int group) { return group >= 1; }

hipError_t launch_zero_f32(float *p, int n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    zero_kernel<<<(n + 255) / 256, 256, 0, stream>>>(p, n);
    return hipGetLastError();
}

size_t bwd_workspace_bytes(int T, int hq, int hkv, int window)
{
    (void)hkv;
    (void)window;
    const size_t delta = ((size_t)hq * T * sizeof(float) + 255) & ~(size_t)255;
    return delta + 256;
}

hipError_t launch_bwd(const BwdArgs &A, hipStream_t stream)
{
    const LayerArgs &a = A.L;
    const long rows = (long)a.T * a.hq;
    const long pre_blocks = (rows + 63) / 64;
    if (pre_blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    trace_begin("bwd_pre", stream);
    bwd_pre_kernel<<<(unsigned)pre_blocks, 256, 0, stream>>>(A);
    trace_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (A.dsink) {
        trace_begin("bwd_dsink", stream);
        if (a.T > 0) bwd_dsink_kernel<<<a.hq, 256, 0, stream>>>(A);
        else zero_kernel<<<(a.hq + 255) / 256, 256, 0, stream>>>(A.dsink, a.hq);
        trace_end(stream);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long kv_tiles = (long)(a.T + NKB - 1) / NKB + a.batch;
    const long kv_grid = kv_tiles * a.hkv;
    if (kv_grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    trace_begin(a.window >= 0 ? "bwd_dkdv_swa" : "bwd_dkdv_global", stream);
    if (a.window >= 0) bwd_dkdv_kernel<true><<<(unsigned)kv_grid, 256, 0, stream>>>(A);
    else bwd_dkdv_kernel<false><<<(unsigned)kv_grid, 256, 0, stream>>>(A);
    trace_end(stream);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int G = a.hq / a.hkv;
    if (G % 8 == 0) return launch_dq<8>(A, stream);
    if (G % 4 == 0) return launch_dq<4>(A, stream);
    if (G % 2 == 0) return launch_dq<2>(A, stream);
    return launch_dq<1>(A, stream);
}

}  // namespace mimo
