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
// up to split_len rows) and walks it in 32-row chunks.  Each chunk's K and V rows are copied HBM -> LDS by
// direct-to-LDS loads whose 64 lanes cover whole rows (coalesced: the rows of one KV head are 1.5 KB
// apart in the cache); S^T = K q^T takes K rows from LDS as MFMA A operands (the G query heads of the
// group are the MFMA columns) and O^T = V^T P^T reads V transposed.  One 20 KB buffer per workgroup and
// at most 256 registers per wave (K operands read four ahead of their MFMAs, V operands just before
// theirs) let eight workgroups share a CU, two waves per SIMD: a wave's next chunk is copied while the
// other wave on its SIMD computes, which kept more bytes in flight than two buffers at four workgroups per
// CU or deeper rings with fewer.  Each split writes an unnormalised
// partial (o, running max, running sum); the combine kernel merges the splits with the sink and the new
// token (whose rotation is computed there in double precision).  A sliding-window decode (at most four
// chunks, one split) copies its chunks all at once into four buffers and merges the new token and the
// sink itself, with no combine kernel.  The query's rotation angles depend only on the position and the
// dim, so a decode wave computes each of the 32 once (in double precision) and shares them by lane
// shuffles.  Per chunk, only a chunk that reaches past the split's rows or past some column's visible rows
// evaluates the mask, and the running max is a lazy reference that moves only when a chunk's max exceeds
// it by 2^8, so most chunks skip the rescale of the output accumulator (both wave-uniform branches).
//
// The same kernels serve two more forms.  Paged cache (page size 1: SGLang cookbook page "MiMo-V2.6",
// section 2): cache row r of sequence b is pool row page_table[cu_cache[b] + r]; each lane of the first 32
// holds the pool row of one row of the next chunk, read one chunk ahead, and the copies take per-lane
// addresses.  Verify (speculative decoding's draft tokens, same page): nq query tokens per sequence whose
// keys are already the last nq cache rows (no k_new); the MFMA columns are (token, head) pairs, and each
// column sees the rows up to its own token and at most `window` below it.  With two to four blocks of 32
// columns, verify_split_kernel runs them as the waves of one workgroup over a shared chunk ring.
#include "device_common.hpp"
#include "internal.hpp"

namespace mimo {
namespace {

constexpr int CH = 32;            // cache rows per chunk
constexpr float RESCALE_TH = 8.f; // keep a stale running max until a chunk's max exceeds it by 2^8

__device__ __forceinline__ double inv_freq(double base, int d) { return pow(base, -(double)d / (double)NHALF); }

// LDS buffer of a decode wave: chunk of CH cache rows of one KV head, K rows (chunk q of row r at
// swz384(r, q): conflict-free 16-row operand reads) and V rows (chunk q at swz256t(r, q): conflict-free
// transposed reads).
constexpr int DKC = DQK / 8;      // 16-byte chunks per K row (24)
constexpr int DVC = DVV / 8;      // per V row (16)
struct DecTile {
    uint4 k[CH * DKC];
    uint4 v[CH * DVC];
};

// A pointer the whole wave holds the same value of, moved to scalar registers (the DMA base operand must
// be scalar; the compiler cannot always prove uniformity through the chunk loop).
__device__ __forceinline__ const u16 *wave_uniform(const u16 *p)
{
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const u16 *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// NB = 1: one buffer, chunks copied and computed in turn (see the loop).  NB = 4 (decode over a window of
// at most four chunks, one split): all chunks are copied at once, so the workgroup waits for one HBM round
// trip instead of four, and with FIN it also merges the new token and the sink and writes the output, so no
// combine kernel follows.
template <bool PAGED, int NB, bool FIN>
__global__ __launch_bounds__(64, 2) void decode_split_kernel(const DecodeArgs A)
{
    __shared__ __attribute__((aligned(256))) DecTile ring[NB];
    const int lane = threadIdx.x, hh = lane >> 5, c = lane & 31;
    const int grp = lane >> 4, t4 = (lane & 15) >> 2, m4 = lane & 3;
    const int G = A.hq / A.hkv;
    // query columns of a KV head: (query token, head) pairs, token-major; decode has one query token per
    // sequence, verify A.nq draft tokens whose keys are already the last A.nq cache rows (no k_new)
    const bool verify = A.k_new == nullptr;
    const int NC = G * A.nq;
    const int ngrp = (NC + 31) / 32;         // the columns in blocks of 32 MFMA columns
    // workgroup order: KV head fastest, so that the one-wave workgroups of a row range's KV heads are
    // dispatched together and the heads' slices of each cache row (one contiguous run) are fetched together
    int w = blockIdx.x;
    const int kvh = w % A.hkv;
    w /= A.hkv;
    const int split = w % A.splits;
    w /= A.splits;
    const int hgrp = w % ngrp;
    const int b = w / ngrp;
    if (b >= A.batch) return;

    int c0 = __builtin_amdgcn_readfirstlane(A.cu_cache[b]);
    const int c1 = __builtin_amdgcn_readfirstlane(A.cu_cache[b + 1]);
    // rows that some query of the sequence can see: decode the last `window` (the new token comes on top),
    // verify the last window + nq (the first draft token's window reaches window rows below it)
    const int keep = verify ? A.window + A.nq : A.window;
    if (A.window >= 0 && c1 - c0 > keep) c0 = c1 - keep;
    const int n = c1 - c0;
    const int ks = split * A.split_len;
    const int ke = min(n, ks + A.split_len);
    const int gi = hgrp * 32 + c;            // this lane's column
    const bool hvalid = gi < NC;
    const int gcol = hvalid ? gi : NC - 1;   // spare MFMA columns repeat the last column
    const int ti = gcol / G;                 // query token of the column
    const int h = kvh * G + gcol % G;
    const size_t part = (((size_t)b * A.nq + ti) * A.hq + h) * A.splits + split;
    // rows this column may see (indices from c0): decode all; verify those up to its own token (row
    // n - nq + ti) and at most `window` below it
    int lim = n - 1, lo = 0;
    if (verify) {
        lim = n - A.nq + ti;
        lo = A.window >= 0 ? lim - A.window : min(lim, 0);
    }
    // rows that every column of the wave may see: [lo_max, lim_min] (wave-uniform)
    const int lim_min = verify ? n - A.nq : n - 1;
    const int lo_max = verify && A.window >= 0 ? n - 1 - A.window : 0;

    if (!FIN && ks >= ke) {                  // nothing cached in this split: an empty partial
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

    // ---- the split's cache rows stream HBM -> LDS (coalesced 16-byte chunks of whole rows, fixed per-lane
    // offsets from a wave-uniform chunk base); rows past the split's end are clamped to its last row
    const size_t krow = (size_t)A.hkv * DQK, vrow = (size_t)A.hkv * DVV;
    uint32_t koff[CH * DKC / 64], voff[CH * DVC / 64];
#pragma unroll
    for (int j = 0; j < CH * DKC / 64; ++j) {
        const int slot = 64 * j + lane, r = slot / DKC, q = slot % DKC;
        koff[j] = (uint32_t)((r * krow + 8 * swz384(r, q)) * 2);
    }
#pragma unroll
    for (int j = 0; j < CH * DVC / 64; ++j) {
        const int slot = 64 * j + lane, r = slot / DVC, q = slot % DVC;
        voff[j] = (uint32_t)((r * vrow + 8 * swz256t(r, q)) * 2);
    }
    const int klast = ks + (ke - ks - 1) / CH * CH;   // first row of the split's last chunk
    // paged cache: pool rows of the chunk's cache rows, lane r (mod 32) holding row k + r (clamped to the
    // split's end); read one chunk ahead of its copy
    auto table_rows = [&](int k) __attribute__((always_inline)) {
        k = min(k, klast);
        return A.page_table[c0 + min(k + c, ke - 1)];
    };
    int tv = PAGED && ks < ke ? table_rows(ks) : 0;
    auto issue = [&](int k, DecTile &T) __attribute__((always_inline)) {
        k = __builtin_amdgcn_readfirstlane(min(k, klast));   // past the end: the last chunk again (uniform waits)
        if constexpr (PAGED) {
#pragma unroll
            for (int j = 0; j < CH * DKC / 64; ++j) {
                const int slot = 64 * j + lane, r = slot / DKC, q = slot % DKC;
                const int row = __shfl(tv, r, 64);
                lds_dma16_nt(A.k_cache + ((size_t)row * A.hkv + kvh) * DQK + 8 * swz384(r, q), T.k + 64 * j);
            }
#pragma unroll
            for (int j = 0; j < CH * DVC / 64; ++j) {
                const int slot = 64 * j + lane, r = slot / DVC, q = slot % DVC;
                const int row = __shfl(tv, r, 64);
                lds_dma16_nt(A.v_cache + ((size_t)row * A.hkv + kvh) * DVV + 8 * swz256t(r, q), T.v + 64 * j);
            }
            tv = table_rows(k + CH);
        } else if (k + CH <= ke) {
            const u16 *kb = wave_uniform(A.k_cache + ((size_t)(c0 + k) * A.hkv + kvh) * DQK);
            const u16 *vb = wave_uniform(A.v_cache + ((size_t)(c0 + k) * A.hkv + kvh) * DVV);
#pragma unroll
            for (int j = 0; j < CH * DKC / 64; ++j) lds_dma16_nt(kb, koff[j], T.k + 64 * j);
#pragma unroll
            for (int j = 0; j < CH * DVC / 64; ++j) lds_dma16_nt(vb, voff[j], T.v + 64 * j);
        } else {
#pragma unroll
            for (int j = 0; j < CH * DKC / 64; ++j) {
                const int slot = 64 * j + lane, r = slot / DKC, q = slot % DKC;
                const int row = c0 + min(k + r, ke - 1);
                lds_dma16_nt(A.k_cache + ((size_t)row * A.hkv + kvh) * DQK + 8 * swz384(r, q), T.k + 64 * j);
            }
#pragma unroll
            for (int j = 0; j < CH * DVC / 64; ++j) {
                const int slot = 64 * j + lane, r = slot / DVC, q = slot % DVC;
                const int row = c0 + min(k + r, ke - 1);
                lds_dma16_nt(A.v_cache + ((size_t)row * A.hkv + kvh) * DVV + 8 * swz256t(r, q), T.v + 64 * j);
            }
        }
    };
    if constexpr (NB == 1) {
        if (ks < ke) issue(ks, ring[0]);
    } else if (ks < ke) {
        // all NB chunks at once (the split's last chunk again past its end); paged: the pool rows of every
        // chunk are read first, so the copies do not wait on table loads issued between them
        int tvs[NB];
        if constexpr (PAGED) {
#pragma unroll
            for (int i = 0; i < NB; ++i) tvs[i] = table_rows(ks + CH * i);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if constexpr (PAGED) tv = tvs[i];
            issue(ks + CH * i, ring[i]);
        }
    }

    // rotated query (bf16) as the B operand: column = head, dims 16s + 8hh + t.  FIN: also this lane's part
    // of the new token's score, q' . k_new' with k_new rotated at the same position in fp32
    bf16x8 qf[12];
    float dot_new = 0.f;
    {
        const u16 *qp = A.q + (((size_t)b * A.nq + ti) * A.hq + h) * DQK + 8 * hh;
#pragma unroll
        for (int s = 0; s < 12; ++s) qf[s] = ld16(qp + 16 * s);
        const double pos = (double)A.positions[b] + (double)ti;
        // decode: every column sits at the sequence's position, so the 32 angles of the rotated dims are
        // computed once (lane l takes dim l % 32) and each lane fetches the 16 it uses; verify columns sit at
        // their own draft positions and compute theirs
        float cf = 0.f, sf = 0.f;
        if (!verify) {
            double sn, cn;
            sincos(pos * inv_freq(A.rope_base, lane & 31), &sn, &cn);
            cf = (float)cn;
            sf = (float)sn;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float2 cs[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (!verify) {
                    const int d = 16 * s + 8 * hh + t;
                    cs[t] = make_float2(__shfl(cf, d, 64), __shfl(sf, d, 64));
                } else {
                    double sn, cn;
                    sincos(pos * inv_freq(A.rope_base, 16 * s + 8 * hh + t), &sn, &cn);
                    cs[t] = make_float2((float)cn, (float)sn);
                }
            }
            rope_pair(qf[s], qf[s + 2], cs);
            if constexpr (FIN) {
                const u16 *kp = A.k_new + ((size_t)b * A.hkv + kvh) * DQK + 8 * hh;
                const bf16x8 k0 = ld16(kp + 16 * s), k1 = ld16(kp + 16 * (s + 2));
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float a0 = bf2f(k0[t]), a1 = bf2f(k1[t]);
                    dot_new += bf2f(qf[s][t]) * (a0 * cs[t].x - a1 * cs[t].y) +
                               bf2f(qf[s + 2][t]) * (a1 * cs[t].x + a0 * cs[t].y);
                }
            }
        }
        if constexpr (FIN) {
            const u16 *kp = A.k_new + ((size_t)b * A.hkv + kvh) * DQK + 8 * hh;
#pragma unroll
            for (int s = 4; s < 12; ++s) {
                const bf16x8 k0 = ld16(kp + 16 * s);
#pragma unroll
                for (int t = 0; t < 8; ++t) dot_new += bf2f(qf[s][t]) * bf2f(k0[t]);
            }
        }
        // every q register is complete before the chunk loop: otherwise the compiler's own load waits for
        // them, placed inside the loop, also stall on the cache loads in flight
#pragma unroll
        for (int s = 0; s < 12; ++s) asm volatile("" : "+v"(qf[s]));
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x16{};

    // transposed V read r of k-step s covers rows 16 s + 8 r + 4 hh + t4 and columns 32 i + 16 (grp & 1)
    // + 4 m4 .. + 3 (the order in which the score registers hold the keys)
    auto vtr = [&](const DecTile &T, int s, int r, int i) __attribute__((always_inline)) -> const char * {
        const int R = 16 * s + 8 * r + 4 * hh + t4;
        const int q = 4 * i + 2 * (grp & 1) + (m4 >> 1);
        return (const char *)T.v + R * (DVC * 16) + 16 * swz256t(R, q) + 8 * (m4 & 1);
    };
    auto chunk = [&](int k, const DecTile &T) __attribute__((always_inline)) {
        constexpr int KR = 4;             // K operands read ahead of their MFMA (a ring: fewer registers)
        auto kread = [&](int s) __attribute__((always_inline)) {
            return ld16((const u16 *)T.k + (c * DKC + swz384(c, 2 * s + hh)) * 8);
        };
        bf16x8 kop[KR];
#pragma unroll
        for (int s = 0; s < KR; ++s) kop[s] = kread(s);
        f32x16 sacc = f32x16{};
#pragma unroll
        for (int s = 0; s < 12; ++s) {
            sacc = mfma32(kop[s % KR], qf[s], sacc);
            if (s + KR < 12) kop[s % KR] = kread(s + KR);
        }
        // only a chunk that reaches past the split's rows or past some column's visible rows evaluates the
        // mask (a wave-uniform branch)
        float mx = -INFINITY;
        if (!(k + CH <= ke && k + CH - 1 <= lim_min && k >= lo_max)) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = k + 8 * (j >> 2) + 4 * hh + (j & 3);
                const bool ok = key < ke && (uint32_t)(key - lo) <= (uint32_t)(lim - lo);
                sacc[j] = ok ? sacc[j] : -INFINITY;
            }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[j]);
        mx = pair_max(mx) * A.scale_log2;
        // lazy reference: it moves only when the chunk's max exceeds it by 2^8 (probabilities stay below 2^8),
        // so most chunks skip the rescale of o and l (exact either way: numerator and denominator share it)
        const bool grow = mx > m_run + RESCALE_TH;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            // (lanes that do not grow keep alpha = 1: their m_run may still be -inf)
            const float alpha = grow ? fast_exp2(m_run - mx) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] *= alpha;
            m_run = grow ? mx : m_run;
        }
        // a verify column may see none of the keys so far: keep it at (max -inf, sum 0) without NaNs
        const float nref = m_run == -INFINITY ? 0.f : -m_run;
        float psum = 0.f;
        bf16x8 pf[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float pj = fast_exp2(__builtin_fmaf(sacc[j], A.scale_log2, nref));
            psum += pj;
            pf[j >> 3][j & 7] = f2bf(pj);
        }
        l_run += psum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x8 v0 = tr_pair(vtr(T, 0, 0, i), vtr(T, 0, 1, i));
            const bf16x8 v1 = tr_pair(vtr(T, 1, 0, i), vtr(T, 1, 1, i));
            o[i] = mfma32(v0, pf[0], o[i]);
            o[i] = mfma32(v1, pf[1], o[i]);
        }
    };

    if constexpr (NB == 1) {
        // ---- one buffer: wait for chunk k (the only loads in flight), compute it, wait until every LDS read
        // of the buffer has returned, then copy chunk k + CH into it (the other wave on the SIMD computes
        // meanwhile)
        for (int k = ks; k < ke; k += CH) {
            wait_vmcnt<0>();
            chunk(k, ring[0]);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // every read of the buffer has returned
            if (k + CH < ke) issue(k + CH, ring[0]);
        }
    } else if (ks < ke) {
        // ---- every chunk in flight: chunk i has landed once at most the copies of the later ones are
        // outstanding (each chunk is CH * (DKC + DVC) / 64 copy instructions, issued in order)
        constexpr int LC = CH * (DKC + DVC) / 64;
        static_assert(NB == 4, "the waits below are written for four chunks");
        wait_vmcnt<3 * LC>();
        chunk(ks, ring[0]);
        wait_vmcnt<2 * LC>();
        if (ks + CH < ke) chunk(ks + CH, ring[1]);
        wait_vmcnt<LC>();
        if (ks + 2 * CH < ke) chunk(ks + 2 * CH, ring[2]);
        wait_vmcnt<0>();
        if (ks + 3 * CH < ke) chunk(ks + 3 * CH, ring[3]);
    }
    wait_vmcnt<0>();                        // no load may still target this workgroup's LDS at exit

    const float l_tot = pair_sum(l_run);
    if constexpr (FIN) {
        // ---- the new token's score (q' . k_new' with k_new rotated at the same position, in fp32) and the
        // sink join the running max and sum, then out = 0.707 * o / sum in bf16
        const float s_new = pair_sum(dot_new) * A.scale_log2;
        const float sk = A.sink ? A.sink[h] * LOG2E : -INFINITY;
        const float M = fmaxf(fmaxf(m_run, s_new), sk);
        const float alpha = fast_exp2(m_run - M), w_new = fast_exp2(s_new - M);
        const float Lt = l_tot * alpha + w_new + (sk > -INFINITY ? fast_exp2(sk - M) : 0.f);
        const float inv = VSCALE / Lt;
        const u16 *vp = A.v_new + ((size_t)b * A.hkv + kvh) * DVV + 4 * hh;
        u16 *out = A.out + (((size_t)b * A.nq + ti) * A.hq + h) * DVV + 4 * hh;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const bf16x4 v4 = __builtin_bit_cast(bf16x4, *(const uint2 *)(vp + 32 * i + 8 * jj));
                bf16x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = f2bf((o[i][4 * jj + t] * alpha + w_new * bf2f(v4[t])) * inv);
                if (hvalid) *(uint2 *)(out + 32 * i + 8 * jj) = __builtin_bit_cast(uint2, w);
            }
        return;
    }
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

// Verify with several blocks of 32 (draft token, head) columns: one workgroup of VNW waves per (sequence,
// KV head, split), one wave per column block, all sharing one LDS ring of VNB chunks, so each chunk is
// copied once for all column blocks (the one-wave form copies it once per block).  Two such workgroups
// share a CU (76 KB of LDS and at most 256 registers per wave), so a SIMD holds two waves whose softmax
// and MFMA work interleave; that mattered more than a deeper ring at one workgroup per CU (8 draft tokens x
// 16 heads: 3.8 ms against 6.4 ms with six chunks, 9.0 ms in the one-wave form).
constexpr int VNW = 4;            // waves (column blocks) per verify workgroup
constexpr int VNB = 3;            // chunks in the shared ring (60 KB; two in flight)
constexpr int VTAB = 4096;        // paged: the split's pool rows staged in LDS (splits longer than this use
                                  // the one-wave form)

template <bool PAGED>
__global__ __launch_bounds__(64 * VNW, 2) void verify_split_kernel(const DecodeArgs A)
{
    __shared__ __attribute__((aligned(256))) DecTile ring[VNB];
    __shared__ __attribute__((aligned(16))) int32_t stab[PAGED ? VTAB : 1];
    const int lane = threadIdx.x & 63, hh = lane >> 5, c = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 4, t4 = (lane & 15) >> 2, m4 = lane & 3;
    const int G = A.hq / A.hkv;
    // query columns of a KV head: (query token, head) pairs, token-major; decode has one query token per
    // sequence, verify A.nq draft tokens whose keys are already the last A.nq cache rows (no k_new)
    const bool verify = A.k_new == nullptr;
    const int NC = G * A.nq;
    const int ngrp = (NC + 31) / 32;         // the columns in blocks of 32 MFMA columns
    (void)ngrp;                              // one wave per block of 32 columns (at most VNW blocks)
    // workgroup order: KV head fastest (the heads' slices of each cache row are fetched together)
    int w = blockIdx.x;
    const int kvh = w % A.hkv;
    w /= A.hkv;
    const int split = w % A.splits;
    const int hgrp = wave;
    const int b = w / A.splits;
    if (b >= A.batch) return;

    int c0 = __builtin_amdgcn_readfirstlane(A.cu_cache[b]);
    const int c1 = __builtin_amdgcn_readfirstlane(A.cu_cache[b + 1]);
    // rows that some query of the sequence can see: decode the last `window` (the new token comes on top),
    // verify the last window + nq (the first draft token's window reaches window rows below it)
    const int keep = verify ? A.window + A.nq : A.window;
    if (A.window >= 0 && c1 - c0 > keep) c0 = c1 - keep;
    const int n = c1 - c0;
    const int ks = split * A.split_len;
    const int ke = min(n, ks + A.split_len);
    const int gi = hgrp * 32 + c;            // this lane's column
    const bool hvalid = gi < NC;
    const int gcol = hvalid ? gi : NC - 1;   // spare MFMA columns repeat the last column
    const int ti = gcol / G;                 // query token of the column
    const int h = kvh * G + gcol % G;
    const size_t part = (((size_t)b * A.nq + ti) * A.hq + h) * A.splits + split;
    // rows this column may see (indices from c0): decode all; verify those up to its own token (row
    // n - nq + ti) and at most `window` below it
    int lim = n - 1, lo = 0;
    if (verify) {
        lim = n - A.nq + ti;
        lo = A.window >= 0 ? lim - A.window : min(lim, 0);
    }
    // rows that every column of the wave may see: [lo_max, lim_min] (wave-uniform)
    const int lim_min = verify ? n - A.nq : n - 1;
    const int lo_max = verify && A.window >= 0 ? n - 1 - A.window : 0;

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

    // ---- the split's cache rows stream HBM -> LDS (coalesced 16-byte chunks of whole rows, fixed per-lane
    // offsets from a wave-uniform chunk base); rows past the split's end are clamped to its last row
    const size_t krow = (size_t)A.hkv * DQK, vrow = (size_t)A.hkv * DVV;
    constexpr int KJ = CH * DKC / 64 / VNW, VJ = CH * DVC / 64 / VNW;   // this wave's slots: j = VNW jj + wave
    static_assert(KJ * VNW * 64 == CH * DKC && VJ * VNW * 64 == CH * DVC, "slot split");
    uint32_t koff[KJ], voff[VJ];
#pragma unroll
    for (int jj = 0; jj < KJ; ++jj) {
        const int slot = 64 * (VNW * jj + wave) + lane, r = slot / DKC, q = slot % DKC;
        koff[jj] = (uint32_t)((r * krow + 8 * swz384(r, q)) * 2);
    }
#pragma unroll
    for (int jj = 0; jj < VJ; ++jj) {
        const int slot = 64 * (VNW * jj + wave) + lane, r = slot / DVC, q = slot % DVC;
        voff[jj] = (uint32_t)((r * vrow + 8 * swz256t(r, q)) * 2);
    }
    const int klast = ks + (ke - ks - 1) / CH * CH;   // first row of the split's last chunk
    // paged cache: the split's pool rows are staged in LDS once (a compiler-visible load inside the chunk
    // loop would make the compiler wait for every copy in flight before using it)
    if constexpr (PAGED) {
        for (int i = threadIdx.x; i < ke - ks; i += 64 * VNW) stab[i] = A.page_table[c0 + ks + i];
        __syncthreads();
    }
    // one chunk: this wave's share of its copy (KJ K slots and VJ V slots per lane), whole rows per
    // instruction; past the split's end the last chunk again, so every wave issues the same number of loads
    auto issue = [&](int k, DecTile &T) __attribute__((always_inline)) {
        k = __builtin_amdgcn_readfirstlane(min(k, klast));
        if constexpr (PAGED) {
#pragma unroll
            for (int jj = 0; jj < KJ; ++jj) {
                const int j = VNW * jj + wave, slot = 64 * j + lane, r = slot / DKC, q = slot % DKC;
                const int row = stab[min(k + r, ke - 1) - ks];
                lds_dma16_nt(A.k_cache + ((size_t)row * A.hkv + kvh) * DQK + 8 * swz384(r, q), T.k + 64 * j);
            }
#pragma unroll
            for (int jj = 0; jj < VJ; ++jj) {
                const int j = VNW * jj + wave, slot = 64 * j + lane, r = slot / DVC, q = slot % DVC;
                const int row = stab[min(k + r, ke - 1) - ks];
                lds_dma16_nt(A.v_cache + ((size_t)row * A.hkv + kvh) * DVV + 8 * swz256t(r, q), T.v + 64 * j);
            }
        } else if (k + CH <= ke) {
            const u16 *kb = wave_uniform(A.k_cache + ((size_t)(c0 + k) * A.hkv + kvh) * DQK);
            const u16 *vb = wave_uniform(A.v_cache + ((size_t)(c0 + k) * A.hkv + kvh) * DVV);
#pragma unroll
            for (int jj = 0; jj < KJ; ++jj) lds_dma16_nt(kb, koff[jj], T.k + 64 * (VNW * jj + wave));
#pragma unroll
            for (int jj = 0; jj < VJ; ++jj) lds_dma16_nt(vb, voff[jj], T.v + 64 * (VNW * jj + wave));
        } else {
#pragma unroll
            for (int jj = 0; jj < KJ; ++jj) {
                const int j = VNW * jj + wave, slot = 64 * j + lane, r = slot / DKC, q = slot % DKC;
                const int row = c0 + min(k + r, ke - 1);
                lds_dma16_nt(A.k_cache + ((size_t)row * A.hkv + kvh) * DQK + 8 * swz384(r, q), T.k + 64 * j);
            }
#pragma unroll
            for (int jj = 0; jj < VJ; ++jj) {
                const int j = VNW * jj + wave, slot = 64 * j + lane, r = slot / DVC, q = slot % DVC;
                const int row = c0 + min(k + r, ke - 1);
                lds_dma16_nt(A.v_cache + ((size_t)row * A.hkv + kvh) * DVV + 8 * swz256t(r, q), T.v + 64 * j);
            }
        }
    };

    // rotated query (bf16) as the B operand: column = head, dims 16s + 8hh + t
    bf16x8 qf[12];
    {
        const u16 *qp = A.q + (((size_t)b * A.nq + ti) * A.hq + h) * DQK + 8 * hh;
#pragma unroll
        for (int s = 0; s < 12; ++s) qf[s] = ld16(qp + 16 * s);
        const double pos = (double)A.positions[b] + (double)ti;
        // the angles depend only on (token, dim): when this wave's 32 columns span at most two draft tokens
        // (16 or more heads per KV head), lane l computes token t_lo + l / 32, dim l % 32 once (in double
        // precision) and each lane fetches the 16 it uses; otherwise every lane computes its own
        const int t_lo = hgrp * 32 / G, t_hi = min(hgrp * 32 + 31, NC - 1) / G;
        const bool shared = t_hi - t_lo <= 1;
        float cf = 0.f, sf = 0.f;
        if (shared) {
            double sn, cn;
            sincos(((double)A.positions[b] + (double)(t_lo + (lane >> 5))) * inv_freq(A.rope_base, lane & 31), &sn, &cn);
            cf = (float)cn;
            sf = (float)sn;
        }
        const int src0 = 32 * (ti - t_lo);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float2 cs[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (shared) {
                    const int d = src0 + 16 * s + 8 * hh + t;
                    cs[t] = make_float2(__shfl(cf, d, 64), __shfl(sf, d, 64));
                } else {
                    double sn, cn;
                    sincos(pos * inv_freq(A.rope_base, 16 * s + 8 * hh + t), &sn, &cn);
                    cs[t] = make_float2((float)cn, (float)sn);
                }
            }
            rope_pair(qf[s], qf[s + 2], cs);
        }
        // every q register is complete before the chunk loop: otherwise the compiler's own load waits for
        // them, placed inside the loop, also stall on the cache loads in flight
#pragma unroll
        for (int s = 0; s < 12; ++s) asm volatile("" : "+v"(qf[s]));
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x16{};

    // transposed V read r of k-step s covers rows 16 s + 8 r + 4 hh + t4 and columns 32 i + 16 (grp & 1)
    // + 4 m4 .. + 3 (the order in which the score registers hold the keys)
    auto vtr = [&](const DecTile &T, int s, int r, int i) __attribute__((always_inline)) -> const char * {
        const int R = 16 * s + 8 * r + 4 * hh + t4;
        const int q = 4 * i + 2 * (grp & 1) + (m4 >> 1);
        return (const char *)T.v + R * (DVC * 16) + 16 * swz256t(R, q) + 8 * (m4 & 1);
    };
    auto chunk = [&](int k, const DecTile &T) __attribute__((always_inline)) {
        bf16x8 kop[12];
#pragma unroll
        for (int s = 0; s < 12; ++s) kop[s] = ld16((const u16 *)T.k + (c * DKC + swz384(c, 2 * s + hh)) * 8);
        f32x16 sacc = f32x16{};
#pragma unroll
        for (int s = 0; s < 12; ++s) sacc = mfma32(kop[s], qf[s], sacc);
        bf16x8 vop[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) vop[m] = tr_pair(vtr(T, m & 1, 0, m >> 1), vtr(T, m & 1, 1, m >> 1));
        // only a chunk that reaches past the split's rows or past some column's visible rows evaluates the
        // mask (a wave-uniform branch)
        float mx = -INFINITY;
        if (!(k + CH <= ke && k + CH - 1 <= lim_min && k >= lo_max)) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = k + 8 * (j >> 2) + 4 * hh + (j & 3);
                const bool ok = key < ke && (uint32_t)(key - lo) <= (uint32_t)(lim - lo);
                sacc[j] = ok ? sacc[j] : -INFINITY;
            }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[j]);
        mx = pair_max(mx) * A.scale_log2;
        // lazy reference: it moves only when the chunk's max exceeds it by 2^8 (probabilities stay below 2^8),
        // so most chunks skip the rescale of o and l (exact either way: numerator and denominator share it)
        const bool grow = mx > m_run + RESCALE_TH;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            // (lanes that do not grow keep alpha = 1: their m_run may still be -inf)
            const float alpha = grow ? fast_exp2(m_run - mx) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] *= alpha;
            m_run = grow ? mx : m_run;
        }
        // a verify column may see none of the keys so far: keep it at (max -inf, sum 0) without NaNs
        const float nref = m_run == -INFINITY ? 0.f : -m_run;
        float psum = 0.f;
        bf16x8 pf[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float pj = fast_exp2(__builtin_fmaf(sacc[j], A.scale_log2, nref));
            psum += pj;
            pf[j >> 3][j & 7] = f2bf(pj);
        }
        l_run += psum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[i] = mfma32(vop[2 * i], pf[0], o[i]);
            o[i] = mfma32(vop[2 * i + 1], pf[1], o[i]);
        }
    };

    // ---- ring of VNB buffers shared by the waves, VNB - 1 chunks in flight: at chunk i wait until this
    // wave's part of it landed (the newer chunks may stay in flight), barrier (every wave's part landed and
    // every wave finished chunk i - 1), refill chunk i - 1's buffer with chunk i + VNB - 1, compute chunk i
    const int nch = (ke - ks + CH - 1) / CH;
#pragma unroll
    for (int i = 0; i < VNB - 1; ++i) issue(ks + i * CH, ring[i]);
    for (int i = 0; i < nch; ++i) {
        wait_vmcnt<(VNB - 2) * (KJ + VJ)>();
        __builtin_amdgcn_s_barrier();
        issue(ks + (i + VNB - 1) * CH, ring[(i + VNB - 1) % VNB]);
        chunk(ks + i * CH, ring[i % VNB]);
    }
    wait_vmcnt<0>();                        // no load may still target this workgroup's LDS at exit

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

// One workgroup of NWV waves per (sequence, query head): merge the splits, the new token and the sink.
// Wave w takes splits w, w + NWV, ...; the partial sums are added in wave order (deterministic).  Four
// waves when there are many splits (a small batch over long caches), one otherwise.
template <int NWV>
__global__ __launch_bounds__(64 * NWV) void decode_combine_kernel(const DecodeArgs A)
{
    __shared__ float red_m[NWV], red_l[NWV];
    __shared__ float2 red_o[NWV][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x / A.hq, h = blockIdx.x % A.hq;   // row = b * nq + query token
    const int b = row / A.nq;
    const int G = A.hq / A.hkv, kvh = h / G;
    const double pos = (double)A.positions[b];
    const bool verify = A.k_new == nullptr;   // verify: the queries' own keys are cache rows already

    // score of the new token (decode): rotate q and k_new in fp32 from fp64 angles
    const u16 *qp = A.q + ((size_t)row * A.hq + h) * DQK;
    const u16 *kp = verify ? nullptr : A.k_new + ((size_t)b * A.hkv + kvh) * DQK;
    float dot = 0.f;
    if (!verify && lane < NHALF) {
        double sn, cn;
        sincos(pos * inv_freq(A.rope_base, lane), &sn, &cn);
        const float cf = (float)cn, sf = (float)sn;
        const float q0 = bf2f(__builtin_bit_cast(__bf16, qp[lane])), q1 = bf2f(__builtin_bit_cast(__bf16, qp[lane + 32]));
        const float k0 = bf2f(__builtin_bit_cast(__bf16, kp[lane])), k1 = bf2f(__builtin_bit_cast(__bf16, kp[lane + 32]));
        const float qa = q0 * cf - q1 * sf, qb = q1 * cf + q0 * sf;
        const float ka = k0 * cf - k1 * sf, kb = k1 * cf + k0 * sf;
        dot = qa * ka + qb * kb;
    }
    if (!verify)
        for (int d = 64 + lane; d < DQK; d += 64)
            dot += bf2f(__builtin_bit_cast(__bf16, qp[d])) * bf2f(__builtin_bit_cast(__bf16, kp[d]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
    const float s_new = verify ? -INFINITY : dot * A.scale_log2;

    // common reference: the largest of the new score, the sink and every split's max
    const float *ml = A.part_ml + ((size_t)row * A.hq + h) * A.splits * 2;
    const float *po = A.part_o + ((size_t)row * A.hq + h) * A.splits * DVV;
    const float sk = A.sink ? A.sink[h] * LOG2E : -INFINITY;
    float M = fmaxf(s_new, sk);
    for (int s = tid; s < A.splits; s += 64 * NWV) M = fmaxf(M, ml[2 * s]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    if (NWV > 1) {
        if (lane == 0) red_m[wave] = M;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NWV; ++w) M = fmaxf(M, red_m[w]);
    }

    // this wave's splits: weighted sums of the partial numerators (dims 2 lane, 2 lane + 1) and denominators
    float L = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll 4
    for (int s = wave; s < A.splits; s += NWV) {
        const float m = ml[2 * s];
        const float wgt = m == -INFINITY ? 0.f : fast_exp2(m - M);
        L += wgt * ml[2 * s + 1];
        const float2 x = *(const float2 *)(po + (size_t)s * DVV + 2 * lane);
        o0 += wgt * x.x;
        o1 += wgt * x.y;
    }
    red_o[wave][lane] = make_float2(o0, o1);
    if (lane == 0) red_l[wave] = L;
    __syncthreads();
    if (wave != 0) return;
    float t0 = 0.f, t1 = 0.f, w_new = 0.f;
    if (!verify) {
        w_new = fast_exp2(s_new - M);
        const u16 *vp = A.v_new + ((size_t)b * A.hkv + kvh) * DVV;
        t0 = w_new * bf2f(__builtin_bit_cast(__bf16, vp[2 * lane]));
        t1 = w_new * bf2f(__builtin_bit_cast(__bf16, vp[2 * lane + 1]));
    }
    float Lt = w_new + (sk > -INFINITY ? fast_exp2(sk - M) : 0.f);
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        Lt += red_l[w];
        t0 += red_o[w][lane].x;
        t1 += red_o[w][lane].y;
    }
    const float inv = VSCALE / Lt;
    u16 *out = A.out + ((size_t)row * A.hq + h) * DVV + 2 * lane;
    out[0] = __builtin_bit_cast(u16, f2bf(t0 * inv));
    out[1] = __builtin_bit_cast(u16, f2bf(t1 * inv));
}

}  // namespace

bool decode_group_supported(int group) { return group >= 1; }

void decode_split_plan(int batch, int max_cache_len, int hq, int hkv, int window, int *splits, int *split_len)
{
    (void)hq;
    (void)hkv;
    int n = max_cache_len;
    if (window >= 0 && window < n) n = window;
    // up to 32 splits per sequence at a batch of 64 and proportionally more for smaller batches (a batch
    // of one long cache still fills the chip: 1024 splits of 1024 rows at 1M rows), each a multiple of the
    // chunk and at least 1024 rows
    const int target = batch >= 64 ? 32 : min(1024, 32 * ((64 + max(batch, 1) - 1) / max(batch, 1)));
    int len = (n + target - 1) / target;
    len = (len + CH - 1) / CH * CH;
    if (len < 1024) len = 1024;
    int s = (n + len - 1) / len;
    if (s < 1) s = 1;
    *splits = s;
    *split_len = len;
}

static size_t partials_bytes(int batch, int nq, int hq, int splits)
{
    const size_t po = ((size_t)batch * nq * hq * splits * DVV * sizeof(float) + 255) & ~(size_t)255;
    const size_t ml = (size_t)batch * nq * hq * splits * 2 * sizeof(float);
    return po + ml;
}

size_t decode_workspace_bytes(int batch, int max_cache_len, int hq, int window, int nq)
{
    int splits, len;
    decode_split_plan(batch, max_cache_len, hq, 1, window, &splits, &len);
    return partials_bytes(batch, nq, hq, splits);
}

bool decode_split_plan_capped(int batch, int max_cache_len, int hq, int window, int nq, size_t cap, int *splits,
                              int *split_len)
{
    decode_split_plan(batch, max_cache_len, hq, 1, window, splits, split_len);
    if (partials_bytes(batch, nq, hq, *splits) <= cap) return true;
    if (partials_bytes(batch, nq, hq, 1) > cap) return false;
    // the most splits that fit, then chunk-aligned lengths that cover the visible rows with at most that many
    const size_t per = (size_t)batch * nq * hq * (DVV + 2) * sizeof(float);
    const int smax = (int)((cap - 255) / per);
    int n = max_cache_len;
    if (window >= 0 && window < n) n = window;
    int len = (n + smax - 1) / smax;
    len = (len + CH - 1) / CH * CH;
    if (len < *split_len) len = *split_len;
    *split_len = len;
    *splits = n > 0 ? (n + len - 1) / len : 1;
    return partials_bytes(batch, nq, hq, *splits) <= cap;
}

hipError_t launch_decode(const DecodeArgs &A, hipStream_t stream)
{
    const int G = A.hq / A.hkv;
    const long waves = (long)A.batch * A.hkv * ((G * A.nq + 31) / 32) * A.splits;
    if (waves > 0x7fffffffL || (long)A.batch * A.nq * A.hq > 0x7fffffffL) return hipErrorInvalidConfiguration;
    trace_begin(A.window >= 0 ? "decode_split_swa" : "decode_split_global", stream);
    const int ngrp = (G * A.nq + 31) / 32;
    if (A.k_new == nullptr && ngrp > 1 && ngrp <= VNW && (!A.page_table || A.split_len <= VTAB)) {
        const unsigned wgs = (unsigned)((long)A.batch * A.hkv * A.splits);
        if (A.page_table) verify_split_kernel<true><<<wgs, 64 * VNW, 0, stream>>>(A);
        else verify_split_kernel<false><<<wgs, 64 * VNW, 0, stream>>>(A);
    } else {
        // decode over a window of at most four chunks (one split): the chunks are copied all at once and the
        // split kernel writes the output itself
        const bool fin = A.k_new != nullptr && A.splits == 1 && A.window >= 0 && A.window <= 4 * CH;
        if (A.page_table) {
            if (fin) decode_split_kernel<true, 4, true><<<(unsigned)waves, 64, 0, stream>>>(A);
            else decode_split_kernel<true, 1, false><<<(unsigned)waves, 64, 0, stream>>>(A);
        } else {
            if (fin) decode_split_kernel<false, 4, true><<<(unsigned)waves, 64, 0, stream>>>(A);
            else decode_split_kernel<false, 1, false><<<(unsigned)waves, 64, 0, stream>>>(A);
        }
        if (fin) {
            trace_end(stream);
            return hipGetLastError();
        }
    }
    trace_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    trace_begin("decode_combine", stream);
    const unsigned rows = (unsigned)((long)A.batch * A.nq * A.hq);
    if (A.splits > 16) decode_combine_kernel<4><<<rows, 256, 0, stream>>>(A);
    else decode_combine_kernel<1><<<rows, 64, 0, stream>>>(A);
    trace_end(stream);
    return hipGetLastError();
}

}  // namespace mimo
