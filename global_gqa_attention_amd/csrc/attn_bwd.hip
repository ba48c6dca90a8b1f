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
//   1. bwd_pre:   D and LSE * log2(e) for every (head, token), zero-padded to T_pad; a block owns 16 tokens
//                 x 16 heads, so each head's 16 values are written together.
//   2. bwd_dsink: one 1024-thread workgroup per head, fixed-order tree sum (only when a sink is given).
//   3. row_prep:  DMA-ready copies in the workspace: q' (rotated) row-major, k' (rotated) row-major and
//                 transposed (the transposed copy keeps each 16-token group's 4-token chunks in the order
//                 (0, 2, 1, 3), the order in which the score registers hold tokens).  Not run for q when the
//                 forward's rotated q is given, nor for k when its rotated k is given on the stored-dS path.
//   4. bwd_dkdv:  key-major.  A workgroup owns 128 keys of one KV head (32 per wave; the key is the MFMA
//                 column, so each lane owns one key with its rotated k and v resident in registers) and
//                 walks every (query head of the group, 32-query tile) that sees them: S = Q'K'^T and
//                 dP = dO V^T, P and dS, then dV^T += dO^T P and dK^T += Q'^T dS.  The q' and dO row tiles and
//                 LSE/D stream HBM -> LDS with global_load_lds (three-stage ring, XOR-swizzled); the
//                 transposed operands of dV and dK come from the same tiles through ds_read_b64_tr_b16.
//                 Causal layers walk query tiles outer and the workgroup's heads inner; with a window the
//                 two halves of the key tile each walk only the tiles their keys see, one tile each per
//                 stage.  With the stored-dS workspace it also writes every dS block it computes.
//   5. bwd_dq:    either from the stored dS blocks (5b: dQ^T += K'^T dS^T, no recomputation; one query tile of
//                 up to sixteen heads per workgroup, which share each k' tile), or
//                 query-major like the forward: S^T = K'Q'^T, P^T, dP^T = V dO^T, dS^T, then
//                 dQ^T += K'^T dS^T with k' (both layouts) and v streamed HBM -> LDS.
// dq and dk leave through the transposed rotation in their epilogues.  Rows that a lane owns (the dK/dV score
// waves' k' and v at the start; dq, dk, dv and the fp32 partials at the end) move between HBM and the lanes
// through LDS that is idle at that moment, so that each memory instruction covers whole rows instead of one
// 16-byte piece of each of 32 rows.
#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"

namespace mimo {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float RSQRT_DQK = 0.07216878364870322f;   // 1 / sqrt(192)

__device__ __forceinline__ int seq_start_of(const int32_t *cu, int batch, int t)
{
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return cu[lo];
}

// column of token t inside its 16-token group in the transposed copies: 4-token chunks (0, 2, 1, 3)
__device__ __forceinline__ int tperm16(int t)
{
    const int c4 = (t >> 2) & 3;
    return (t & ~15) | ((((c4 & 1) << 1) | (c4 >> 1)) << 2) | (t & 3);
}

// ------------------------------------------------------------------------------------------------------
// Stored-dS layout.  A block is 32 queries x 32 keys of one head in bf16 (2 KB), written by the dK/dV
// kernel in its own register order as two 1 KB planes: plane P, row (L ^ 8 (L / 32) ^ 4 P) holds the 8
// values of lane L = key + 32 hh for queries 16 P + 4 hh + 8 (e / 4) + e % 4, e = 0..7 (the row permutation
// spreads the dQ kernel's transposed reads over all LDS banks; each plane is one whole store).  Query tiles of sequence b
// start at S16 = seq_start & ~15 (tile n: S16 + 32 n ..), key blocks at seq_start (block k: seq_start +
// 32 k ..).  Row n of a sequence holds the key blocks k_lo(n) .. k_hi(n) that tile n sees: causal rows
// have n + 1 slots, sliding-window rows ds_row_width(window) slots.  Slot s of all sequences' rows is
// numbered ds_index[b] + rows before n + (k - k_lo(n)), and the query heads are the innermost index: block
// (slot, h) sits at slot * hq + h, so the dQ kernel's NH heads of one step read one contiguous run.
// ------------------------------------------------------------------------------------------------------
__host__ __device__ __forceinline__ int ds_row_width(int window) { return (window + 62) / 32 + 1; }
__device__ __forceinline__ int ds_nq(int seq_start, int seq_end)
{
    return seq_end > seq_start ? (seq_end - 1 - (seq_start & ~15)) / 32 + 1 : 0;
}
__device__ __forceinline__ int64_t ds_rows_before(int n, int window)
{
    return window >= 0 ? (int64_t)n * ds_row_width(window) : (int64_t)n * (n + 1) / 2;
}
// first key block that query tile n (first query q0) can see
__device__ __forceinline__ int ds_klo(int q0, int seq_start, int window)
{
    return window >= 0 ? max(0, q0 - window - seq_start) / 32 : 0;
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
// 1. D = rowsum(dO * O) and LSE * log2(e), both [hq, T_pad] with zero padding
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdArgs A)
{
    // a block owns 16 tokens x 16 heads: per token the 16 heads' dO and O rows are one contiguous run (a
    // 16-lane group per row), and D and LSE*log2(e) of a head are written as 16 consecutive values
    __shared__ float sd[16][17];
    const int tid = threadIdx.x, g = tid >> 4, sub = tid & 15;
    const int t0 = blockIdx.x * 16, h = blockIdx.y * 16 + g;
    const int T = A.L.T, hq = A.L.hq;
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
        const int t = t0 + it;
        float s = 0.f;
        if (t < T && h < hq) {
            const size_t r = (size_t)t * hq + h;
            const bf16x8 x = ld16_nt(A.dout + r * DVV + 8 * sub);
            const bf16x8 y = ld16_nt(A.out + r * DVV + 8 * sub);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += bf2f(x[e]) * bf2f(y[e]);
        }
        s += __shfl_xor(s, 8, 16);
        s += __shfl_xor(s, 4, 16);
        s += __shfl_xor(s, 2, 16);
        s += __shfl_xor(s, 1, 16);
        if (sub == 0) sd[g][it] = s;
    }
    __syncthreads();
    if (h < hq) {
        const int t = t0 + sub;
        A.delta[(size_t)h * A.T_pad + t] = sd[g][sub];
        A.lse2[(size_t)h * A.T_pad + t] = t < T ? A.lse[(size_t)h * T + t] * LOG2E : 0.f;
    }
}

// ------------------------------------------------------------------------------------------------------
// 2. dsink_h = -sum_t exp(sink_h - LSE_t) D_t, fixed order
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void bwd_dsink_kernel(const BwdArgs A)
{
    // one workgroup per head: each thread sums a fixed stride of tokens, then the wave sums (shuffle tree)
    // and the 16 wave totals in wave order
    __shared__ float red[16];
    const int h = blockIdx.x, tid = threadIdx.x;
    const float sk = A.L.sink[h];
    float acc = 0.f;
    if (sk > -INFINITY) {
        const float *lse = A.lse + (size_t)h * A.L.T, *dl = A.delta + (size_t)h * A.T_pad;
#pragma unroll 4
        for (int t = tid; t < A.L.T; t += 1024) acc -= expf(sk - lse[t]) * dl[t];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if ((tid & 63) == 0) red[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < 16; ++w) s += red[w];
        A.dsink[h] = s;
    }
}

__global__ void zero_kernel(float *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// ds_index[b] = dS blocks of sequences 0 .. b-1 within one head (exclusive scan over the batch, one
// workgroup), ds_index[batch] = blocks per head
__global__ __launch_bounds__(256) void bwd_ds_index_kernel(const BwdArgs A)
{
    __shared__ int64_t part[256];
    const int tid = threadIdx.x, batch = A.L.batch;
    const int per = (batch + 255) / 256, b0 = min(batch, tid * per), b1 = min(batch, b0 + per);
    auto region = [&](int b) { return ds_rows_before(ds_nq(A.L.cu[b], A.L.cu[b + 1]), A.L.window); };
    int64_t sum = 0;
    for (int b = b0; b < b1; ++b) sum += region(b);
    part[tid] = sum;
    __syncthreads();
    if (tid == 0) {
        int64_t run = 0;
        for (int i = 0; i < 256; ++i) {
            const int64_t v = part[i];
            part[i] = run;
            run += v;
        }
        A.ds_index[batch] = run;
    }
    __syncthreads();
    int64_t run = part[tid];
    for (int b = b0; b < b1; ++b) {
        A.ds_index[b] = run;
        run += region(b);
    }
}

// ------------------------------------------------------------------------------------------------------
// 3. row_prep: for 64 tokens of head h of x [T, H, D]: optional rotation of dims 0..63, then a row-major
//    copy rm [T_pad, H, D] and/or a transposed copy tr [H, D, T_pad] (tokens in tperm16 order), zero-filled
//    for tokens T .. T_pad-1.
// ------------------------------------------------------------------------------------------------------
template <int D, bool ROPE>
__global__ __launch_bounds__(256) void row_prep_kernel(const u16 *x, int H, u16 *rm, u16 *tr, LayerArgs a, int T_pad)
{
    __shared__ __attribute__((aligned(16))) u16 sX[64 * (D + 8)];
    constexpr int CH = D / 8;
    const int tid = threadIdx.x, h = blockIdx.x % H, t0 = (blockIdx.x / H) * 64;   // heads fastest
    // load (and rotate) 64 rows: thread handles row tid/4, chunks cg, cg+4, cg+8, ...
    {
        const int rr = tid >> 2, cg = tid & 3, t = t0 + rr;
        bf16x8 v[CH / 4];
        const u16 *src = x + ((size_t)t * H + h) * D;
#pragma unroll
        for (int i = 0; i < CH / 4; ++i)
            v[i] = t < a.T ? ld16_nt(src + 8 * (cg + 4 * i)) : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        if (ROPE && t < a.T) {
            const int pos = t - seq_start_of(a.cu, a.batch, t);
            const float2 *cs = a.rope + (size_t)min(pos, a.rope_len - 1) * NHALF + 8 * cg;
            float2 c8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) c8[e] = cs[e];
            rope_pair(v[0], v[1], c8);     // chunks cg and cg + 4: dims d and d + 32
        }
#pragma unroll
        for (int i = 0; i < CH / 4; ++i) {
            st16(sX + rr * (D + 8) + 8 * (cg + 4 * i), v[i]);
            if (rm && t < T_pad) st16(rm + ((size_t)t * H + h) * D + 8 * (cg + 4 * i), v[i]);
        }
    }
    if (!tr) return;
    __syncthreads();
    // transposed rows: D dims x 8 chunks of 8 tokens
    for (int item = tid; item < D * 8; item += 256) {
        const int d = item >> 3, cc = item & 7;
        if (t0 + 8 * cc >= T_pad) continue;
        bf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = __builtin_bit_cast(__bf16, sX[tperm16(8 * cc + e) * (D + 8) + d]);
        st16(tr + ((size_t)h * D + d) * T_pad + t0 + 8 * cc, w);
    }
}

// ------------------------------------------------------------------------------------------------------
// 4. dK, dV (key-major)
// ------------------------------------------------------------------------------------------------------
constexpr int NKB = 128;                 // keys per workgroup (four 32-key blocks)
constexpr int MQ = 32;                   // queries per step
constexpr int QCH = DQK / 8;             // 24 chunks per q' row
constexpr int OCH = DVV / 8;             // 16 chunks per dO row
constexpr int DK_AHEAD = 4;              // LDS operand reads in flight ahead of the MFMAs

struct DkdvTile {
    uint4 qr[MQ * QCH], orow[MQ * OCH];  // q' and dO rows (read as rows and, transposed, as columns)
    float ld[2 * MQ];                    // LSE * log2(e) [MQ], then D [MQ]
};

// Eight waves, two per 32-key block.  Score wave kb (0..3) holds the keys' k' and v and computes S and dP
// from the row tiles, then P and dS; gradient wave 4 + kb holds dV and dK and, one step later, takes P and
// dS (bf16) from the score wave through LDS for dV^T += dO^T P and dK^T += Q'^T dS (transposed operands).
// Each wave holds half the state, so two waves fit on a SIMD and interleave: the score wave's softmax
// and dS VALU run under the gradient wave's MFMAs.
template <bool WIN>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(const BwdArgs A)
{
    const LayerArgs &a = A.L;
    // tiles of stages st-1, st, st+1 (sliding window: a ring of three for each half of the keys, ring[3 g + k];
    // each half's three tiles lie within 64 KB, the reach of an LDS instruction's offset field)
    __shared__ __attribute__((aligned(16))) DkdvTile ring[WIN ? 6 : 3];
    __shared__ __attribute__((aligned(16))) uint4 pbuf[2][4][256];     // P and dS (bf16) of a step: 4 planes x 64 lanes
    __shared__ __attribute__((aligned(16))) uint4 kstage_own[WIN ? 1 : 4 * 32 * QCH];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int role = wave >> 2, kq = wave & 3;
    const int hh = lane >> 5, c = lane & 31;
    const int G = a.hq / a.hkv;

    // ---- work item: KV head fastest, then head split, then key tiles of the sequences from last to first
    const int x = blockIdx.x;
    const int kvh = x % a.hkv;
    const int split = (x / a.hkv) % A.splits;
    const int GS = G / A.splits;      // query heads handled by this workgroup
    const SeqPos sp = seq_lookup_rev(a.cu, a.batch, x / a.hkv / A.splits, [](int s, int e) { return (e - s + NKB - 1) / NKB; });
    if (sp.b < 0) return;
    const int seq_start = sp.start, seq_end = sp.end, bseq = sp.b, tile = sp.j;
    const int kb0 = seq_start + tile * NKB;
    const int kb_last = min(kb0 + NKB - 1, seq_end - 1);

    // ---- query steps: tiles of 32 queries from kb0 (aligned down to 16: the stored-dS row layout)
    const int q_lo = kb0 & ~15;
    const int q_hi = WIN ? min(seq_end - 1, kb_last + a.window) : seq_end - 1;
    const int nq = (q_hi - q_lo + MQ) / MQ;
    const int q_top = q_lo + (nq - 1) * MQ;
    // Sliding window: the two halves of the key tile (waves 0, 1: keys kb0 .. kb0 + 63; waves 2, 3: the rest)
    // see query ranges 64 apart, so in a stage each half takes a tile of its own: of the tiles counted from
    // the top, half g walks only jlo_g .. jlo_g + n_g - 1, the ones that its keys see, and a head takes as many
    // stages as the half with more tiles (about six instead of eight or nine with a 128-key window, in which
    // a 32-key block sees five tiles).  Causal layers: both halves walk all nq tiles together.
    const int half_g = (wave & 3) >> 1;   // this wave's half of the keys (both roles)
    int nS = nq, qb_g = q_top, n_g = nq;    // stages per head; the half's first tile (its q0) and tile count
    if constexpr (WIN) {
        auto half = [&](int kg0, int &lo, int &n) {
            if (kg0 > kb_last) {
                lo = 0;
                n = 0;
                return;
            }
            const int kg1 = min(kg0 + 63, kb_last);
            // tile j (first query q_top - 32 j) is seen iff q0 <= kg1 + window and q0 + 31 >= kg0
            lo = max(0, (q_top - kg1 - a.window + MQ - 1) >> 5);
            const int hi = min(nq - 1, (q_top + MQ - 1 - kg0) >> 5);
            n = max(0, hi - lo + 1);
        };
        int lo0, n0, lo1, n1;
        half(kb0, lo0, n0);
        half(kb0 + 64, lo1, n1);
        nS = max(n0, n1);
        qb_g = q_top - MQ * (half_g ? lo1 : lo0);
        n_g = half_g ? n1 : n0;
    }
    const int nsteps = nS * GS;

    // ---- direct HBM -> LDS loads of one step's tiles (fixed per-lane byte offsets + wave-uniform bases):
    // all by the gradient waves (4..7), which finish their MFMAs early in each stage, so that the score
    // waves (the kernel's critical path) issue no loads: q' rows three 16-byte chunks per lane, dO rows two,
    // LSE*log2e by wave 6 and D by wave 7 (eight lanes each)
    const size_t qr_row = (size_t)a.hq * DQK, o_row = (size_t)a.hq * DVV;
    const int gw = wave & 3;
    // Sliding window: each half's tile is loaded by that half's two gradient waves (4, 5 and 6, 7), so chunk
    // slot 128 j + 64 (wave & 1) + lane; slots 384 (q') and 256 (dO) further on are the rows 16 further on,
    // which have the same swizzle, so the per-lane offsets of j serve j + 3 (q') and j + 2 (dO) as well.
    const int gslot = WIN ? 64 * (wave & 1) : 64 * gw, gstride = WIN ? 128 : 256;
    uint32_t o_qr[3], o_or[2];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int slot = gstride * j + gslot + lane, r = slot / QCH, p = slot % QCH;
        o_qr[j] = (uint32_t)((r * qr_row + 8 * swz384t(r, p)) * 2);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int slot = gstride * j + gslot + lane, r = slot / OCH, p = slot % OCH;
        o_or[j] = (uint32_t)((r * o_row + 8 * swz256t(r, p)) * 2);
    }
    // Causal step -> (query tile, head): query tiles from the sequence end down, the workgroup's heads inner.
    // Every key tile of a sequence walks the same absolute query tiles in the same order from the top, so
    // the workgroups running together on an XCD stay on the same q'/dO tiles (a key tile nearer the end of
    // the sequence only stops earlier) and mostly hit in L2.  The stages walk the steps in order, so the
    // position advances by one head per stage (no division per stage).  (Sliding window: see below.)
    struct Pos {
        int q0, h;   // first query of the step's tile, its query head
    };
    const Pos first{q_top, kvh * G + split * GS};
    const int h_end = first.h + GS;
    auto advance = [&](Pos p) {
        ++p.h;
        const bool wrap = p.h == h_end;
        p.h = wrap ? first.h : p.h;
        p.q0 = wrap ? p.q0 - MQ : p.q0;
        return p;
    };
    auto issue = [&](Pos ps, DkdvTile &T) {
        const int h = ps.h, q0 = ps.q0;
        if (q0 + MQ <= A.qr_rows) {
            const u16 *bq = A.W.qr + ((size_t)q0 * a.hq + h) * DQK;
#pragma unroll
            for (int j = 0; j < 3; ++j) lds_dma16(bq, o_qr[j], T.qr + 256 * j + 64 * gw);
        } else {
            // a caller's q_rot has exactly T rows: rows past its end are clamped to the last (and masked)
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int slot = 256 * j + 64 * gw + lane, r = slot / QCH, p = slot % QCH;
                const int row = min(q0 + r, A.qr_rows - 1);
                lds_dma16(A.W.qr + ((size_t)row * a.hq + h) * DQK + 8 * swz384t(r, p), T.qr + 256 * j + 64 * gw);
            }
        }
        if (q0 + MQ <= a.T) {
            const u16 *bo = A.dout + ((size_t)q0 * a.hq + h) * DVV;
#pragma unroll
            for (int j = 0; j < 2; ++j) lds_dma16(bo, o_or[j], T.orow + 256 * j + 64 * gw);
        } else {
            // dO is not padded: rows past its end are clamped to the last row (and masked)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int slot = 256 * j + 64 * gw + lane, r = slot / OCH, p = slot % OCH;
                const int row = min(q0 + r, a.T - 1);
                lds_dma16(A.dout + (size_t)row * o_row + (size_t)h * DVV + 8 * swz256t(r, p), T.orow + 256 * j + 64 * gw);
            }
        }
        if (wave >= 6) {
            const float *bld = (wave == 6 ? A.lse2 : A.delta) + (size_t)h * A.T_pad + q0;
            if (lane < 8) lds_dma16(bld, (uint32_t)(16 * lane), (uint4 *)T.ld + 8 * (wave - 6));
        }
    };
    // sliding window: one half's tile by its two gradient waves (LSE*log2e by the first, D by the second)
    // The tile's LDS address is passed through an empty asm so that the compiler forms each copy's m0 value
    // next to its copy instead of keeping all of them (eleven per tile, three ring slots) in scalar registers.
    auto issue_w = [&](Pos ps, DkdvTile &T) {
        const int h = ps.h, q0 = ps.q0;
        uint32_t tb = (uint32_t)(uintptr_t)(lds_void *)&T + 16 * gslot;
        asm volatile("" : "+s"(tb));
        constexpr uint32_t OQ = offsetof(DkdvTile, qr), OO = offsetof(DkdvTile, orow), OL = offsetof(DkdvTile, ld);
        if (q0 + MQ <= A.qr_rows) {
            const u16 *bq = A.W.qr + ((size_t)q0 * a.hq + h) * DQK;
#pragma unroll
            for (int j = 0; j < 3; ++j) lds_dma16_m0(bq, o_qr[j], tb + OQ + 16 * 128 * j);
#pragma unroll
            for (int j = 0; j < 3; ++j) lds_dma16_m0(bq + 16 * qr_row, o_qr[j], tb + OQ + 16 * 128 * (j + 3));
        } else {
            // rows past the end (rare): lane laundered so that these per-lane addresses are formed here, not
            // kept in registers across the loop
            int ln = lane;
            asm volatile("" : "+v"(ln));
#pragma unroll
            for (int j = 0; j < 6; ++j) {
                const int slot = 128 * j + gslot + ln, r = slot / QCH, p = slot % QCH;
                const int row = min(q0 + r, A.qr_rows - 1);
                lds_dma16(A.W.qr + ((size_t)row * a.hq + h) * DQK + 8 * swz384t(r, p), T.qr + 128 * j + gslot);
            }
        }
        if (q0 + MQ <= a.T) {
            const u16 *bo = A.dout + ((size_t)q0 * a.hq + h) * DVV;
#pragma unroll
            for (int j = 0; j < 2; ++j) lds_dma16_m0(bo, o_or[j], tb + OO + 16 * 128 * j);
#pragma unroll
            for (int j = 0; j < 2; ++j) lds_dma16_m0(bo + 16 * o_row, o_or[j], tb + OO + 16 * 128 * (j + 2));
        } else {
            int ln = lane;
            asm volatile("" : "+v"(ln));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int slot = 128 * j + gslot + ln, r = slot / OCH, p = slot % OCH;
                const int row = min(q0 + r, a.T - 1);
                lds_dma16(A.dout + (size_t)row * o_row + (size_t)h * DVV + 8 * swz256t(r, p), T.orow + 128 * j + gslot);
            }
        }
        const float *bld = ((wave & 1) == 0 ? A.lse2 : A.delta) + (size_t)h * A.T_pad + q0;
        if (lane < 8) lds_dma16_m0(bld, (uint32_t)(16 * lane), tb - 16 * gslot + OL + 16 * 8 * (wave & 1));
    };

    // ---- this wave's keys
    const int kw0 = kb0 + 32 * kq;
    const int kj = kw0 + c;
    const bool kvalid = kj <= kb_last;
    const int kjl = kvalid ? kj : kb_last;

    // Which queries of a step do these keys need?  None (skip), all (no mask), or some (mask).
    auto visible = [&](int step, Pos ps) {
        const int q0 = ps.q0;
        return step < nsteps && !(q0 + MQ - 1 < kw0 || kw0 > kb_last || (WIN && q0 > kw0 + 31 + a.window));
    };
    auto masked = [&](Pos ps) {
        const int q0 = ps.q0;
        return q0 < kw0 + 31 || q0 + MQ - 1 > q_hi || (WIN && q0 + MQ - 1 - kw0 > a.window) || kw0 + 31 > kb_last;
    };
    // mask bound: query qi sees this lane's key iff 0 <= qi - kj <= ub.  Lanes past the tile's last key see
    // nothing (their key is moved 2^30 away, so the unsigned test fails): their dK/dV are never written back,
    // and their dS blocks must hold zeros.
    const int ub = !kvalid ? 0 : WIN ? min(a.window, q_hi - kj) : q_hi - kj;
    const int kjm = kvalid ? kj : kj + (1 << 30);

    // Transposed operand reads: read r of k-step s covers rows 16 s + 8 r + 4 hh + t4 and the four columns
    // 32 i + 16 (grp & 1) + 4 m4 .. + 3 of the operand's 32-row block i (lane il = 4 t4 + m4).
    const int grp = lane >> 4, t4 = (lane & 15) >> 2, m4 = lane & 3;
    auto tr_at = [&](const void *tile_, int rowbytes, bool w384, int s, int r, int i) -> const char * {
        const int R = 16 * s + 8 * r + 4 * hh + t4;
        const int q = 4 * i + 2 * (grp & 1) + (m4 >> 1);
        const int p = w384 ? swz384t(R, q) : swz256t(R, q);
        return (const char *)tile_ + R * rowbytes + 16 * p + 8 * (m4 & 1);
    };

    // ---- tile ring: at stage st the tiles of steps st (score waves) and st-1 (gradient waves) are read and
    // step st+1 is loaded: a gradient wave waits for its loads (step st's tiles, issued one stage earlier),
    // every wave makes its P / dS writes of the previous stage visible, barrier (every gradient wave has
    // landed its part, every wave has finished stage st-1, so the buffer of step st-2 is free), the
    // gradient waves load step st+1.  Every stage loads one tile set (the last step's again once the steps
    // run out), so the waits stay uniform.  Both roles pass nsteps + 1 barriers.  The score waves' dS
    // stores need no wait (their data registers are the compiler's to protect).
    // pc: step st, pn: step min(st + 1, nsteps - 1) (the one stage st loads)
    Pos pc = first, pn = nsteps > 1 ? advance(first) : first;
    // a gradient wave waits for its loads of step st (issued one stage earlier), every wave makes its LDS
    // writes of the previous stage visible, then the barrier; the gradient waves load step st + 1
    auto stage_start = [&](DkdvTile &fill) {
        if (role == 1) wait_vmcnt<0>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        if (role == 1) issue(pn, fill);
    };
    auto stage_end = [&](int st) {
        pc = pn;
        if (st + 2 <= nsteps - 1) pn = advance(pn);
    };
    // Sliding window: a stage is (j, head), j = 0 .. nS - 1; the half's tile at stage j has q0 = qb_g - 32 j
    // while j < n_g (none after).  Slot k of the ring is ring[k] (keys kb0 .. kb0 + 63) and ring[3 + k]
    // (the rest) -- ring[3 g + k] for half g; a half's tile is loaded only at the stages where it has one.
    struct St {
        int j, h;
    };
    auto st_next = [&](St s) {
        if (++s.j == nS) {
            s.j = 0;
            ++s.h;
        }
        return s;
    };
    auto pos_of = [&](St s) { return Pos{qb_g - MQ * max(0, min(s.j, n_g - 1)), s.h}; };
    St sc{0, first.h};            // stage st
    St sn = st_next(sc);          // stage st + 1 (the one stage st loads)
    auto stage_start_w = [&](int st, DkdvTile &fill) {
        if (role == 1) wait_vmcnt<0>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        if (role == 1 && st + 1 < nsteps && sn.j < n_g) issue_w(pos_of(sn), fill);
    };
    auto stage_end_w = [&]() {
        sc = sn;
        sn = st_next(sn);
    };
    if (role == 1) {
        if constexpr (WIN) {
            if (n_g > 0) issue_w(pos_of(sc), ring[3 * half_g]);
        } else {
            issue(first, ring[0]);
        }
    }

    if (role == 0) {
        // ================= score waves: S = Q'K'^T and dP = dO V^T, then P and dS = P (0.707 dP - D); P and
        // dS (bf16) go to the gradient wave of the same keys through LDS, dS also to the stored-dS blocks
        bf16x8 kf[12], vf[8];
        {
            // the wave's 32 k' and v rows are copied into LDS by whole rows (chunk slot g by instruction
            // g / 64; k' into its staging array, v into the hand-over buffers, which no wave writes before
            // the first stage's barrier), then each lane reads its own row: a lane that loads its own row
            // touches 32 rows per load instruction
            // (sliding window: in the half's ring slots 1 and 2, first filled after the first barrier)
            uint4 *ks = WIN ? (uint4 *)&ring[3 * (kq >> 1) + 1] + 32 * QCH * (kq & 1) : kstage_own + 32 * QCH * kq;
            uint4 *vs = &pbuf[0][0][0] + 32 * OCH * kq;
            const u16 *kbase = A.W.kr + ((size_t)kb0 * a.hkv + kvh) * DQK;
            const u16 *vbase = a.v + ((size_t)kb0 * a.hkv + kvh) * DVV;
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                const int g = 64 * i + lane, rw = g / QCH, row = min(kw0 + rw, kb_last) - kb0;
                lds_dma16(kbase, (uint32_t)((row * a.hkv * DQK + 8 * swz384(rw, g % QCH)) * 2), ks + 64 * i);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int g = 64 * i + lane, rw = g / OCH, row = min(kw0 + rw, kb_last) - kb0;
                lds_dma16(vbase, (uint32_t)((row * a.hkv * DVV + 8 * swz256(rw, g % OCH)) * 2), vs + 64 * i);
            }
            wait_vmcnt<0>();
#pragma unroll
            for (int s = 0; s < 12; ++s) kf[s] = __builtin_bit_cast(bf16x8, ks[QCH * c + swz384(c, 2 * s + hh)]);
#pragma unroll
            for (int s = 0; s < 8; ++s) vf[s] = __builtin_bit_cast(bf16x8, vs[OCH * c + swz256(c, 2 * s + hh)]);
        }
        // operand k: q' rows (S, k < 12), then dO rows (dP, k - 12)
        auto load_op = [&](int k, const DkdvTile &T) -> bf16x8 {
            if (k < 12) return ld16((const u16 *)T.qr + (c * QCH + swz384t(c, 2 * k + hh)) * 8);
            return ld16((const u16 *)T.orow + (c * OCH + swz256t(c, 2 * (k - 12) + hh)) * 8);
        };
        // dS of a step into the stored-dS blocks (query tile n, key block 4 tile + kq; see ds_row_width)
        const int s16 = seq_start & ~15;
        const int kap = 4 * tile + kq;
        const int64_t ds_seq = A.ds ? A.ds_index[bseq] : 0;
        // block index of a position (sliding window: at every step; causal: the first one only, later ones
        // follow by the steps below)
        auto blk_of = [&](Pos ps) -> int64_t {
            const int n = (ps.q0 - s16) >> 5;
            return (ds_seq + ds_rows_before(n, a.window) + (kap - ds_klo(ps.q0, seq_start, a.window))) * a.hq + ps.h;
        };
        // Causal: the block of the next position.  The next head of the same tile is the next block (heads
        // are the innermost index); one query tile down, back at the first head, removes row n of the
        // sequence's rows (n slots) and the GS - 1 heads walked.
        const int64_t blk_top = A.ds ? blk_of(first) : 0;
        auto blk_next = [&](int64_t b, Pos p, Pos np) -> int64_t {
            if (np.q0 == p.q0) return b + 1;
            return b - (int64_t)((p.q0 - s16) >> 5) * a.hq - (GS - 1);
        };
        int64_t bc = blk_top, bn = blk_top;   // blocks of pc and pn
        if (A.ds && nsteps > 1) bn = blk_next(blk_top, first, pn);
        auto store_ds = [&](int64_t blk, const bf16x8 *sb) {
            if (blk >= A.ds_cap) return false;   // only with a max_seqlen below the longest sequence
            // streaming stores (the blocks are read back by another kernel); plane P holds sb[P] of every lane
            // at row (lane ^ 8 hh ^ 4 P): each store writes a whole 1 KB plane
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            u32x4 *dst = (u32x4 *)(A.ds + blk * 1024);
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, sb[0]), dst + (lane ^ (8 * hh)));
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, sb[1]), dst + 64 + (lane ^ (8 * hh) ^ 4));
            return true;
        };
        auto s_step = [&](Pos ps, const DkdvTile &T, uint4 *pslot) {
            const uint32_t uba = masked(ps) ? (uint32_t)ub : 0xffffffffu;
            const int base = ps.q0 - kjm;   // qi - kj of this lane's first row
            constexpr int R = 2 * DK_AHEAD;
            bf16x8 ob[R];
#pragma unroll
            for (int k = 0; k < DK_AHEAD; ++k) ob[k] = load_op(k, T);
            float4 L4[4], D4[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) L4[jj] = *(const float4 *)(T.ld + 8 * jj + 4 * hh);
            f32x16 sacc = f32x16{}, dpacc = f32x16{};
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 12; ++k) {
                sacc = mfma32(ob[k % R], kf[k], sacc);
                ob[(k + DK_AHEAD) % R] = load_op(k + DK_AHEAD, T);
                if ((k & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
            // the dP MFMAs, each followed by two of the sixteen exponentials: VALU work that needs no MFMA
            // result of its own runs while the MFMA does
            float pv[16];
#pragma unroll
            for (int k = 12; k < 20; ++k) {
                dpacc = mfma32(ob[k % R], vf[k - 12], dpacc);
                if (k + DK_AHEAD < 20) ob[(k + DK_AHEAD) % R] = load_op(k + DK_AHEAD, T);
#pragma unroll
                for (int j = 2 * (k - 12); j < 2 * (k - 12) + 2; ++j) {
                    const int jj = j >> 2, t = j & 3;
                    const float Lv = t == 0 ? L4[jj].x : t == 1 ? L4[jj].y : t == 2 ? L4[jj].z : L4[jj].w;
                    pv[j] = fast_exp2(__builtin_fmaf(sacc[j], a.scale_log2, -Lv));
                }
                if (k == 15) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) D4[jj] = *(const float4 *)(T.ld + MQ + 8 * jj + 4 * hh);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (uba != 0xffffffffu) {   // only steps that cross the causal / window / sequence edge
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    pv[j] = (uint32_t)(base + 8 * (j >> 2) + 4 * hh + (j & 3)) <= uba ? pv[j] : 0.f;
            }
            // hand-over planes (1 KB each, lane-major): P (bf16) values 0..7 and 8..15, then dS the same way
            uint32_t pw[8], sw[8];
#pragma unroll
            for (int w = 0; w < 8; ++w)
                pw[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{pv[2 * w], pv[2 * w + 1]}, bf16x2));
            pslot[lane] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
            pslot[64 + lane] = make_uint4(pw[4], pw[5], pw[6], pw[7]);
            float dsv[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int jj = j >> 2, t = j & 3;
                const float Dv = t == 0 ? D4[jj].x : t == 1 ? D4[jj].y : t == 2 ? D4[jj].z : D4[jj].w;
                dsv[j] = pv[j] * __builtin_fmaf(VSCALE, dpacc[j], -Dv);
            }
#pragma unroll
            for (int w = 0; w < 8; ++w)
                sw[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{dsv[2 * w], dsv[2 * w + 1]}, bf16x2));
            const bf16x8 sb[2] = {__builtin_bit_cast(bf16x8, make_uint4(sw[0], sw[1], sw[2], sw[3])),
                                  __builtin_bit_cast(bf16x8, make_uint4(sw[4], sw[5], sw[6], sw[7]))};
            pslot[128 + lane] = make_uint4(sw[0], sw[1], sw[2], sw[3]);
            pslot[192 + lane] = make_uint4(sw[4], sw[5], sw[6], sw[7]);
            if (A.ds) store_ds(bc, sb);
        };
        auto stage = [&](int st, const DkdvTile &cur, DkdvTile &fill) {
            stage_start(fill);
            if (visible(st, pc)) s_step(pc, cur, pbuf[st & 1][kq]);
            // stage_end's position update, with the block indices beside it
            bc = bn;
            if (A.ds && st + 2 <= nsteps - 1) bn = blk_next(bn, pn, advance(pn));
            stage_end(st);
        };
        auto stage_w = [&](int st, int cs, int fs) {
            stage_start_w(st, ring[3 * half_g + fs]);
            if (sc.j < n_g) {
                const Pos ps = pos_of(sc);
                if (visible(st, ps)) {
                    if (A.ds) bc = blk_of(ps);
                    s_step(ps, ring[3 * half_g + cs], pbuf[st & 1][kq]);
                }
            }
            stage_end_w();
        };
        // unrolled by three: the ring's buffers by name (stage st reads ring[st % 3], fills ring[(st+1) % 3])
        if constexpr (WIN) {
            for (int st = 0; st <= nsteps; st += 3) {
                stage_w(st, 0, 1);
                if (st + 1 > nsteps) break;
                stage_w(st + 1, 1, 2);
                if (st + 2 > nsteps) break;
                stage_w(st + 2, 2, 0);
            }
        } else {
            for (int st = 0; st <= nsteps; st += 3) {
                stage(st, ring[0], ring[1]);
                if (st + 1 > nsteps) break;
                stage(st + 1, ring[1], ring[2]);
                if (st + 2 > nsteps) break;
                stage(st + 2, ring[2], ring[0]);
            }
        }
        wait_vmcnt<0>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();       // the epilogue's barrier (the gradient waves reuse the LDS)
    } else {
        // ================= gradient waves (one step behind): dV^T += dO^T P and dK^T += Q'^T dS, with the
        // transposed operands read from the step's row tiles and P, dS from the score wave of these keys
        f32x16 dv[4], dk[6];
        Pos pg = first;   // step st - 1
#pragma unroll
        for (int i = 0; i < 4; ++i) dv[i] = f32x16{};
#pragma unroll
        for (int i = 0; i < 6; ++i) dk[i] = f32x16{};
        // operand k: dO^T columns (dV, k = 2 i + s), then q'^T columns (dK, k - 8 = 2 i + s)
        auto load_op = [&](int k, const DkdvTile &T) -> bf16x8 {
            if (k < 8) {
                const int i = k >> 1, sk = k & 1;
                return tr_pair(tr_at(T.orow, OCH * 16, false, sk, 0, i), tr_at(T.orow, OCH * 16, false, sk, 1, i));
            }
            const int i = (k - 8) >> 1, sk = (k - 8) & 1;
            return tr_pair(tr_at(T.qr, QCH * 16, true, sk, 0, i), tr_at(T.qr, QCH * 16, true, sk, 1, i));
        };
        auto g_step = [&](const DkdvTile &T, const uint4 *pslot) {
            constexpr int R = 2 * DK_AHEAD;
            bf16x8 ob[R];
#pragma unroll
            for (int k = 0; k < DK_AHEAD; ++k) ob[k] = load_op(k, T);
            bf16x8 pb[2], sb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) pb[i] = __builtin_bit_cast(bf16x8, pslot[64 * i + lane]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 20; ++k) {
                if (k < 8) dv[k >> 1] = mfma32(ob[k % R], pb[k & 1], dv[k >> 1]);
                else dk[(k - 8) >> 1] = mfma32(ob[k % R], sb[(k - 8) & 1], dk[(k - 8) >> 1]);
                if (k + DK_AHEAD < 20) ob[(k + DK_AHEAD) % R] = load_op(k + DK_AHEAD, T);
                if (k == 1) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) sb[i] = __builtin_bit_cast(bf16x8, pslot[128 + 64 * i + lane]);
                }
                if ((k & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto stage = [&](int st, const DkdvTile &prev, DkdvTile &fill) {
            stage_start(fill);
            if (st >= 1 && visible(st - 1, pg)) g_step(prev, pbuf[(st - 1) & 1][kq]);
            pg = pc;
            stage_end(st);
        };
        St sg = sc;   // stage st - 1
        auto stage_w = [&](int st, int ps_, int fs) {
            stage_start_w(st, ring[3 * half_g + fs]);
            if (st >= 1 && sg.j < n_g) {
                const Pos ps = pos_of(sg);
                if (visible(st - 1, ps)) g_step(ring[3 * half_g + ps_], pbuf[(st - 1) & 1][kq]);
            }
            sg = sc;
            stage_end_w();
        };
        // stage st reads ring[(st - 1) % 3] and fills ring[(st + 1) % 3]
        if constexpr (WIN) {
            for (int st = 0; st <= nsteps; st += 3) {
                stage_w(st, 2, 1);
                if (st + 1 > nsteps) break;
                stage_w(st + 1, 0, 2);
                if (st + 2 > nsteps) break;
                stage_w(st + 2, 1, 0);
            }
        } else {
            for (int st = 0; st <= nsteps; st += 3) {
                stage(st, ring[2], ring[1]);
                if (st + 1 > nsteps) break;
                stage(st + 1, ring[0], ring[2]);
                if (st + 2 > nsteps) break;
                stage(st + 2, ring[1], ring[0]);
            }
        }
        wait_vmcnt<0>();
        // ---- epilogue: dv = 0.707 dV^T, dk = R^T dK^T / sqrt(192) (fp32 partials with several head splits).
        // The rows leave through LDS (this wave's 12 KB of the ring for dk, 8 KB of the hand-over buffers for
        // dv, once every wave is past its last read of them): the lanes put their rows in (16-byte chunks
        // XOR-swizzled by row), then each store instruction writes whole rows.
        const float2 *cs = a.rope + (size_t)min(kjl - seq_start, a.rope_len - 1) * NHALF;
        rope_back(dk[0], dk[1], cs, hh);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        uint4 *kst = (uint4 *)ring + kq * 32 * QCH;
        uint4 *vst = &pbuf[0][0][0] + kq * 32 * OCH;
        if (A.splits > 1) {
            // fp32 rows of 48 (dk) + 32 (dv) chunks: two rounds of 16 keys
#pragma unroll
            for (int rd = 0; rd < 2; ++rd) {
                if ((c >> 4) == rd) {
                    const int r = c & 15;
#pragma unroll
                    for (int i = 0; i < 6; ++i)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const int k = 8 * i + 2 * jj + hh;
                            kst[48 * r + ((k & ~15) | ((k & 15) ^ r))] =
                                __builtin_bit_cast(uint4, make_float4(dk[i][4 * jj] * RSQRT_DQK, dk[i][4 * jj + 1] * RSQRT_DQK,
                                                                      dk[i][4 * jj + 2] * RSQRT_DQK, dk[i][4 * jj + 3] * RSQRT_DQK));
                        }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const int k = 8 * i + 2 * jj + hh;
                            vst[32 * r + ((k & ~15) | ((k & 15) ^ r))] =
                                __builtin_bit_cast(uint4, make_float4(dv[i][4 * jj] * VSCALE, dv[i][4 * jj + 1] * VSCALE,
                                                                      dv[i][4 * jj + 2] * VSCALE, dv[i][4 * jj + 3] * VSCALE));
                        }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own rows, read by its lanes
#pragma unroll
                for (int j = 0; j < 12; ++j) {
                    const int g = 64 * j + lane, r = g / 48, p = g % 48, k = (p & ~15) | ((p & 15) ^ r);
                    const int key = kw0 + 16 * rd + r;
                    const uint4 x = kst[g];
                    if (key <= kb_last)
                        *(uint4 *)(A.dkv_part + (((size_t)split * A.T_pad + key) * a.hkv + kvh) * (DQK + DVV) + 4 * k) = x;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int g = 64 * j + lane, r = g >> 5, p = g & 31, k = (p & ~15) | ((p & 15) ^ r);
                    const int key = kw0 + 16 * rd + r;
                    const uint4 x = vst[g];
                    if (key <= kb_last)
                        *(uint4 *)(A.dkv_part + (((size_t)split * A.T_pad + key) * a.hkv + kvh) * (DQK + DVV) + DQK + 4 * k) = x;
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next round's writes
            }
        } else {
            // bf16 rows of 24 (dk) + 16 (dv) chunks
#pragma unroll
            for (int i = 0; i < 6; ++i) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    bf16x4 w;
#pragma unroll
                    for (int t = 0; t < 4; ++t) w[t] = f2bf(dk[i][4 * jj + t] * RSQRT_DQK);
                    const int k = 4 * i + jj;
                    *(uint2 *)((u16 *)(kst + QCH * c + ((k & ~7) | ((k & 7) ^ (c & 7)))) + 4 * hh) = __builtin_bit_cast(uint2, w);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    bf16x4 w;
#pragma unroll
                    for (int t = 0; t < 4; ++t) w[t] = f2bf(dv[i][4 * jj + t] * VSCALE);
                    const int k = 4 * i + jj;
                    *(uint2 *)((u16 *)(vst + OCH * c + (k ^ (c & 15))) + 4 * hh) = __builtin_bit_cast(uint2, w);
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int j = 0; j < 12; ++j) {
                const int g = 64 * j + lane, r = g / QCH, p = g % QCH, k = (p & ~7) | ((p & 7) ^ (r & 7));
                const uint4 x = kst[g];
                if (kw0 + r <= kb_last) st16u_nt(A.dk + ((size_t)(kw0 + r) * a.hkv + kvh) * DQK + 8 * k, x);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int g = 64 * j + lane, r = g >> 4, p = g & 15, k = p ^ (r & 15);
                const uint4 x = vst[g];
                if (kw0 + r <= kb_last) st16u_nt(A.dv + ((size_t)(kw0 + r) * a.hkv + kvh) * DVV + 8 * k, x);
            }
        }
    }
}


// sum of the head-split partials, in split order (deterministic): one thread per 8 of the 320 values
__global__ __launch_bounds__(256) void bwd_dkv_reduce_kernel(const BwdArgs A)
{
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const long rows = (long)A.L.T * A.L.hkv;
    if (idx >= rows * 40) return;
    const long row = idx / 40;
    const int c8 = (int)(idx % 40);
    const int t = (int)(row / A.L.hkv), kvh = (int)(row % A.L.hkv);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int sp = 0; sp < A.splits; ++sp) {
        const float *pp = A.dkv_part + (((size_t)sp * A.T_pad + t) * A.L.hkv + kvh) * (DQK + DVV) + 8 * c8;
        const float4 x0 = *(const float4 *)pp, x1 = *(const float4 *)(pp + 4);
        acc[0] += x0.x; acc[1] += x0.y; acc[2] += x0.z; acc[3] += x0.w;
        acc[4] += x1.x; acc[5] += x1.y; acc[6] += x1.z; acc[7] += x1.w;
    }
    bf16x8 w;
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = f2bf(acc[e]);
    if (c8 < DQK / 8) st16u_nt(A.dk + ((size_t)t * A.L.hkv + kvh) * DQK + 8 * c8, __builtin_bit_cast(uint4, w));
    else st16u_nt(A.dv + ((size_t)t * A.L.hkv + kvh) * DVV + 8 * (c8 - DQK / 8), __builtin_bit_cast(uint4, w));
}

// ------------------------------------------------------------------------------------------------------
// 5. dQ (query-major)
// ------------------------------------------------------------------------------------------------------
constexpr int BN = 32;                   // keys per tile (one step)
constexpr int KCH = DQK / 8;             // 24 chunks per k' row
constexpr int VCH = DVV / 8;             // 16 chunks per v row
constexpr int KTCH = BN / 8;             // 4 chunks per k'^T row
constexpr int DQ_AHEAD = 4;              // LDS operand reads in flight ahead of the MFMAs

struct DqTile {
    uint4 kr[BN * KCH], kt[DQK * KTCH], vr[BN * VCH];
};

template <int NW, int GP, bool WIN>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dq_kernel(const BwdArgs A)
{
    const LayerArgs &a = A.L;
    constexpr int NT = 64 * NW, BM = 32 * NW, TT = BM / GP;
    constexpr int L_KR = BN * KCH / NT, L_KT = DQK * KTCH / NT, L_VR = BN * VCH / NT;
    static_assert(L_KR * NT == BN * KCH && L_KT * NT == DQK * KTCH && L_VR * NT == BN * VCH, "tile split");
    __shared__ __attribute__((aligned(16))) DqTile t0s, t1s, t2s;   // three-stage ring (96 KB)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, c = lane & 31;
    const int G = a.hq / a.hkv;
    const int n_hg = G / GP;

    const int x = blockIdx.x;
    const int kvh = x % a.hkv;
    const int rest = x / a.hkv;
    const int hgi = rest % n_hg;
    const int tile = rest / n_hg;
    const SeqPos sp = seq_lookup_rev(a.cu, a.batch, tile, [](int s, int e) { return (e - s + TT - 1) / TT; });
    if (sp.b < 0) return;
    const int seq_start = sp.start, seq_end = sp.end;
    const int tr = (seq_end - seq_start + TT - 1) / TT - 1 - sp.j;
    const int t0 = seq_start + tr * TT;
    const int t_last = min(t0 + TT - 1, seq_end - 1);
    const int h0 = kvh * G + hgi * GP;

    const int klo = WIN ? max(seq_start, t0 - a.window) : seq_start;
    const int kstart = klo & ~15;
    const int khi = t_last;
    const int nsteps = (khi - kstart + BN) / BN;

    const u16 *kr_g = A.W.kr + (size_t)kvh * DQK, *kt_g = A.W.krt + (size_t)kvh * DQK * A.T_pad;
    const size_t kr_row = (size_t)a.hkv * DQK, v_row = (size_t)a.hkv * DVV;
    uint32_t o_kr[L_KR], o_kt[L_KT], o_vr[L_VR];
#pragma unroll
    for (int j = 0; j < L_KR; ++j) {
        const int slot = NT * j + tid, r = slot / KCH, p = slot % KCH;
        o_kr[j] = (uint32_t)((r * kr_row + 8 * swz384(r, p)) * 2);
    }
#pragma unroll
    for (int j = 0; j < L_KT; ++j) {
        const int slot = NT * j + tid, d = slot / KTCH, p = slot % KTCH;
        o_kt[j] = (uint32_t)(((size_t)d * A.T_pad + 8 * swz64(d, p)) * 2);
    }
#pragma unroll
    for (int j = 0; j < L_VR; ++j) {
        const int slot = NT * j + tid, r = slot / VCH, p = slot % VCH;
        o_vr[j] = (uint32_t)((r * v_row + 8 * swz256(r, p)) * 2);
    }
    auto issue = [&](int step, DqTile &T) {
        const int k0 = kstart + step * BN;
        const u16 *bk = kr_g + (size_t)k0 * kr_row;
        const u16 *bkt = kt_g + k0;
        const u16 *bv = a.v + ((size_t)k0 * a.hkv + kvh) * DVV;
#pragma unroll
        for (int j = 0; j < L_KR; ++j) lds_dma16(bk, o_kr[j], T.kr + NT * j + 64 * wave);
#pragma unroll
        for (int j = 0; j < L_KT; ++j) lds_dma16(bkt, o_kt[j], T.kt + NT * j + 64 * wave);
        if (k0 + BN <= a.T) {
#pragma unroll
            for (int j = 0; j < L_VR; ++j) lds_dma16(bv, o_vr[j], T.vr + NT * j + 64 * wave);
        } else {
            // v is not padded: rows past its end are clamped to the last row (and masked)
#pragma unroll
            for (int j = 0; j < L_VR; ++j) {
                const int slot = NT * j + tid, r = slot / VCH, p = slot % VCH;
                const int row = min(k0 + r, a.T - 1);
                lds_dma16(a.v + (size_t)row * v_row + (size_t)kvh * DVV + 8 * swz256(r, p), T.vr + NT * j + 64 * wave);
            }
        }
    };
    issue(0, t0s);
    issue(min(1, nsteps - 1), t1s);

    // ---- this lane's query row: rotated q and dO as B operands, its LSE and D
    const int r = wave * 32 + c;
    const int qt = t0 + r / GP;
    const int qh = h0 + r % GP;
    const bool qvalid = qt < seq_end;
    const int qtl = qvalid ? qt : t_last;
    bf16x8 qf[12], of[8];
    const float2 *qcs = a.rope + (size_t)min(qtl - seq_start, a.rope_len - 1) * NHALF;
    {
        const u16 *qp = A.W.qr + ((size_t)qtl * a.hq + qh) * DQK + 8 * hh;
#pragma unroll
        for (int s = 0; s < 12; ++s) qf[s] = ld16(qp + 16 * s);
        const u16 *op = A.dout + ((size_t)qtl * a.hq + qh) * DVV + 8 * hh;
#pragma unroll
        for (int s = 0; s < 8; ++s) of[s] = ld16(op + 16 * s);
    }
    const float Lq = A.lse2[(size_t)qh * A.T_pad + qtl];
    const float Dq = A.delta[(size_t)qh * A.T_pad + qtl];

    // this wave's token span and the keys it sees
    const int wt0 = t0 + (wave * 32) / GP;
    const int wt1 = min(t0 + (wave * 32 + 31) / GP, seq_end - 1);
    const int wklo = WIN ? max(seq_start, wt0 - a.window) : seq_start;
    const int wkhi = wt1;
    auto visible = [&](int step) {
        const int k0 = kstart + step * BN;
        return step < nsteps && !(k0 > wkhi || k0 + BN - 1 < wklo);
    };
    auto masked = [&](int step) {
        const int k0 = kstart + step * BN;
        return k0 + BN - 1 > wt0 || k0 < seq_start || (WIN && k0 < wt1 - a.window);
    };
    // mask bound: key kj is seen by this lane's query iff 0 <= qt - kj <= ub (rows of invalid query lanes
    // are never written back)
    const int ub = WIN ? min(a.window, qt - seq_start) : qt - seq_start;

    f32x16 dq[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) dq[i] = f32x16{};

    // S^T = K' Q'^T and dP^T = V dO^T of one tile
    auto sdp = [&](const DqTile &T, f32x16 &sacc, f32x16 &dpacc) {
        const u16 *kr = (const u16 *)T.kr, *vr = (const u16 *)T.vr;
        sacc = f32x16{};
        dpacc = f32x16{};
#pragma unroll
        for (int s = 0; s < 12; ++s) sacc = mfma32(ld16(kr + (c * KCH + swz384(c, 2 * s + hh)) * 8), qf[s], sacc);
#pragma unroll
        for (int s = 0; s < 8; ++s) dpacc = mfma32(ld16(vr + (c * VCH + swz256(c, 2 * s + hh)) * 8), of[s], dpacc);
    };
    // dS^T of one tile (uba = the mask bound, or all-ones for a tile that needs no mask)
    auto softmax = [&](int step, const f32x16 &sacc, const f32x16 &dpacc, uint32_t uba, bf16x8 *sb) {
        const int base = qt - (kstart + step * BN) - 4 * hh;   // qt - key of this lane's first row
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float p = fast_exp2(sacc[j] * a.scale_log2 - Lq);
            p = (uint32_t)(base - 8 * (j >> 2) - (j & 3)) <= uba ? p : 0.f;
            sb[j >> 3][j & 7] = f2bf(p * (VSCALE * dpacc[j] - Dq));
        }
    };
    // dQ^T += K'^T dS^T (two 16-key k-steps)
    auto dq_mm = [&](const DqTile &T, const bf16x8 *sb) {
        const u16 *kt = (const u16 *)T.kt;
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const int d = 32 * i + c;
#pragma unroll
            for (int s = 0; s < 2; ++s) dq[i] = mfma32(ld16(kt + (d * KTCH + swz64(d, 2 * s + hh)) * 8), sb[s], dq[i]);
        }
    };

    // ---- three-stage tile ring, software-pipelined like the dK/dV kernel: at stage st the tiles of steps st
    // and st+1 are read and step st+2 is loaded; the softmax of step st runs between the S/dP products of
    // step st+1, then dQ of step st.
    f32x16 sA = f32x16{}, dA = f32x16{}, sB = f32x16{}, dB = f32x16{};
    wait_vmcnt<L_KR + L_KT + L_VR>();
    __builtin_amdgcn_s_barrier();
    sdp(t0s, sA, dA);
    auto stage = [&](int st, const DqTile &cur, const DqTile &nxt, DqTile &fill, const f32x16 &s0, const f32x16 &d0,
                     f32x16 &s1, f32x16 &d1) {
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        issue(min(st + 2, nsteps - 1), fill);
        if (visible(st) || visible(st + 1)) {
            const uint32_t uba = masked(st) ? (uint32_t)ub : 0xffffffffu;
            bf16x8 sb[2];
            softmax(st, s0, d0, uba, sb);
            sdp(nxt, s1, d1);
            dq_mm(cur, sb);
            __builtin_amdgcn_sched_group_barrier(0x100, DQ_AHEAD, 0);       // first operand reads
#pragma unroll
            for (int i = 0; i < 20; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA (S, dP of step st+1)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          // LDS read
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);          // VALU (softmax of step st)
            }
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA (dQ of step st)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          // LDS read
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);          // VALU
            }
        }
    };
    for (int st = 0; st < nsteps; st += 6) {
        stage(st, t0s, t1s, t2s, sA, dA, sB, dB);
        if (st + 1 >= nsteps) break;
        stage(st + 1, t1s, t2s, t0s, sB, dB, sA, dA);
        if (st + 2 >= nsteps) break;
        stage(st + 2, t2s, t0s, t1s, sA, dA, sB, dB);
        if (st + 3 >= nsteps) break;
        stage(st + 3, t0s, t1s, t2s, sB, dB, sA, dA);
        if (st + 4 >= nsteps) break;
        stage(st + 4, t1s, t2s, t0s, sA, dA, sB, dB);
        if (st + 5 >= nsteps) break;
        stage(st + 5, t2s, t0s, t1s, sB, dB, sA, dA);
    }
    wait_vmcnt<0>();

    // ---- epilogue: dq = R^T dQ^T / sqrt(192).  The rows leave through the idle ring (12 KB per wave, two
    // waves per tile buffer; 16-byte chunks XOR-swizzled by row): the lanes put their rows in, then each
    // store instruction writes whole runs of rows (the GP heads of a token are contiguous)
    rope_back(dq[0], dq[1], qcs, hh);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();           // every wave is done reading the ring
    static_assert(NW <= 4 && sizeof(DqTile) >= 2 * 32 * KCH * sizeof(uint4), "two waves' rows per tile buffer");
    uint4 *stg = (uint4 *)(wave < 2 ? &t0s : &t1s) + (wave & 1) * 32 * KCH;
    {
        u16 *row = (u16 *)(stg + c * KCH) + 4 * hh;
#pragma unroll
        for (int i = 0; i < 6; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = f2bf(dq[i][4 * jj + t] * RSQRT_DQK);
                const int k = 4 * i + jj;
                *(uint2 *)(row + 8 * ((k & ~7) | ((k & 7) ^ (c & 7)))) = __builtin_bit_cast(uint2, w);
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own rows, read by its lanes
#pragma unroll
    for (int j = 0; j < 12; ++j) {
        const int g = 64 * j + lane, rw = g / KCH, p = g % KCH, k = (p & ~7) | ((p & 7) ^ (rw & 7));
        const int r = wave * 32 + rw, tok = t0 + r / GP;
        const uint4 x = stg[g];
        if (tok < seq_end) st16u_nt(A.dq + ((size_t)tok * a.hq + h0 + r % GP) * DQK + 8 * k, x);
    }
}

// ------------------------------------------------------------------------------------------------------
// 5b. dQ from the stored dS blocks: dQ^T += K'^T dS^T per 32-key block, no recomputation.  A workgroup owns
//     one query tile (32 queries) of NH query heads of one KV group (one head per wave) and walks the key
//     blocks the tile sees.  Per block the NH waves share one row-major k' tile (32 keys x 192) and each
//     loads its head's dS block; both MFMA operands come out of LDS through ds_read_b64_tr_b16, which hands
//     every lane of a 16-lane group one 16-bit column element of four rows read by four other lanes:
//     lane i, element t <- the 4-element row read by lane 4 t + i / 4, element i % 4.  The MFMA k index
//     8 hh + 4 r + t of read r (0, 1) stands for key 16 s + 8 r + 4 hh + t in both operands.
// ------------------------------------------------------------------------------------------------------

// NH waves per workgroup, one query head each: the NH heads share every k' tile (the k' rows are loaded
// by the first 768 / 128 = 6 waves, two chunks per lane, or 4 waves, three, when NH = 4; every wave loads
// its own dS block)
template <int NH>
struct DsqTile {
    uint4 kr[32 * KCH];                  // k' rows, 16-byte chunk q of row r at q ^ (4 ((r >> 1) & 1))
    uint4 ds[NH][128];                   // one stored dS block per wave
};

// NS ring stages, OCC workgroups per CU.  Causal layers: all sixteen heads of a KV group per workgroup when
// the group has sixteen (four waves per SIMD, at most 128 registers) and three stages (132 KB), so that each
// k' tile is copied into LDS once per query tile instead of twice (1.93 -> 1.70 ms at the 32K batch); eight
// heads and five stages (140 KB, four block loads in flight) for groups of eight.  Sliding-window layers:
// eight heads (four for groups of four) and two stages (56 KB), two workgroups per CU: their work items are
// short (about six key blocks), and a second resident workgroup hides one's start-up under the other's work
// (four heads, three stages: 0.447 -> 0.414 ms at the 32K batch, against 2.02 ms for 1.95 on the causal
// layer; eight heads, two stages: 0.405 -> 0.367 ms; eight heads, three stages, one workgroup: 0.42 ms).
// Where the ring cannot hold every head's dq rows at once, they leave in two or four rounds.
template <int NH, bool WIN, int NS, int OCC>
__global__ __launch_bounds__(64 * NH, OCC) void bwd_dq_ds_kernel(const BwdArgs A)
{
    const LayerArgs &a = A.L;
    constexpr int KL = NH == 4 ? 3 : 2;                  // k' DMAs per lane of a loading wave
    constexpr int KW = 32 * KCH / (64 * KL);             // waves that load k' (4 or 6)
    __shared__ __attribute__((aligned(16))) DsqTile<NH> ring[NS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, c = lane & 31, grp = lane >> 4, il = lane & 15;
    const int G = a.hq / a.hkv, n_hg = G / NH;

    // ---- work item: KV head fastest, then head group, then query tiles from the last sequence's last tile
    const int x = blockIdx.x;
    const int kvh = x % a.hkv;
    const int hg = (x / a.hkv) % n_hg;
    const SeqPos sp = seq_lookup_rev(a.cu, a.batch, x / a.hkv / n_hg, [](int s, int e) { return ds_nq(s, e); });
    if (sp.b < 0) return;
    const int seq_start = sp.start, seq_end = sp.end, bseq = sp.b;
    const int n = ds_nq(seq_start, seq_end) - 1 - sp.j;
    const int q0 = (seq_start & ~15) + 32 * n;
    const int h = kvh * G + hg * NH + wave;
    const int klo = ds_klo(q0, seq_start, a.window);
    const int khi = min(q0 + 31 - seq_start, seq_end - 1 - seq_start) >> 5;
    const int nsteps = khi - klo + 1;
    const int64_t blk0 = (A.ds_index[bseq] + ds_rows_before(n, a.window)) * a.hq + h;   // step 0's block
    const u16 *ds_row = A.ds + blk0 * 1024;

    // ---- loads of one key block: k' rows (swizzled 16-byte chunks) and this wave's dS block
    const size_t kr_row = (size_t)a.hkv * DQK;
    uint32_t o_kr[KL];
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        const int slot = 64 * KW * j + 64 * min(wave, KW - 1) + lane, r = slot / KCH, p = slot % KCH;
        o_kr[j] = (uint32_t)((r * kr_row + 8 * (p ^ (((r >> 1) & 1) << 2))) * 2);
    }
    auto issue = [&](int step, DsqTile<NH> &T) {
        const int kb = seq_start + 32 * (klo + step);
        const u16 *bk = A.W.kr + ((size_t)kb * a.hkv + kvh) * DQK;
        if (wave < KW) {
            if (kb + 32 <= A.kr_rows) {
#pragma unroll
                for (int j = 0; j < KL; ++j) lds_dma16(bk, o_kr[j], T.kr + 64 * KW * j + 64 * wave);
            } else {
                // a caller's k_rot has exactly T rows: rows past its end are clamped to the last (their dS
                // entries are zero)
#pragma unroll
                for (int j = 0; j < KL; ++j) {
                    const int slot = 64 * KW * j + 64 * wave + lane, r = slot / KCH, p = slot % KCH;
                    const int row = min(kb + r, A.kr_rows - 1);
                    lds_dma16(A.W.kr + ((size_t)row * a.hkv + kvh) * DQK + 8 * (p ^ (((r >> 1) & 1) << 2)),
                              T.kr + 64 * KW * j + 64 * wave);
                }
            }
        }
        // (a block index past the workspace only arises from a max_seqlen below the truth: read block 0)
        const u16 *bd = blk0 + (int64_t)step * a.hq < A.ds_cap ? ds_row + (size_t)step * a.hq * 1024 : A.ds;
        lds_dma16_nt(bd, (uint32_t)(16 * lane), T.ds[wave]);
        lds_dma16_nt(bd, (uint32_t)(16 * (64 + lane)), T.ds[wave] + 64);
    };

    // ---- per-lane parts of the transposed reads.  This lane supplies row (4 hh + t) of a 16-key step for
    // t = il / 4, m = il % 4: k' read r covers dims 32 i + 16 (grp & 1) + 4 m .. + 3 of key 16 s + 8 r + 4 hh +
    // t; the dS read covers queries 16 (grp & 1) + 4 m .. + 3 of that key (row key + 32 (m & 1) of the block,
    // its halves swapped when m & 1).
    const int t4 = il >> 2, m4 = il & 3;
    const int krow = 4 * hh + t4;
    const int ksw = ((krow >> 1) & 1) << 2;
    const int kq = 2 * (grp & 1) + (m4 >> 1);                           // chunk within the 4-chunk block i
    const int a_even = krow * KCH * 16 + ((kq ^ ksw) * 16) + 8 * (m4 & 1);        // dim block i even
    const int a_odd = krow * KCH * 16 + (((4 + kq) ^ ksw) * 16) + 8 * (m4 & 1);   // dim block i odd (i - 1)
    // dS read r of k-step s: plane grp & 1, row (key + 32 hq) ^ 8 hq ^ 4 (grp & 1) with hq = m4 & 1, key =
    // 16 s + 8 r + krow, 8-byte half m4 >> 1 of the 16-byte row
    const int hq_ = m4 & 1, pl = grp & 1;
    const int b_off0 = pl * 1024 + (32 * hq_ + 8 * hq_ + (krow ^ (4 * pl))) * 16 + 8 * (m4 >> 1);
    const int b_off1 = pl * 1024 + (32 * hq_ + 8 * (1 - hq_) + (krow ^ (4 * pl))) * 16 + 8 * (m4 >> 1);

    f32x16 dq[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) dq[i] = f32x16{};

    auto compute = [&](const DsqTile<NH> &T) {
        const char *kb = (const char *)T.kr, *db = (const char *)T.ds[wave];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int rs = 16 * s;   // first key row of the k-step
            const bf16x8 bop = tr_pair(db + b_off0 + rs * 16, db + b_off1 + rs * 16);
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                const int ao = (i & 1 ? a_odd : a_even) + 64 * (i & ~1);
                const bf16x8 aop = tr_pair(kb + ao + rs * KCH * 16, kb + ao + (rs + 8) * KCH * 16);
                dq[i] = mfma32(aop, bop, dq[i]);
            }
        }
    };

    // ---- ring of NS buffers, NS - 1 block loads in flight: at stage st wait until block st landed (the
    // NS - 2 newer sets may still be in flight), barrier (every wave landed its part and finished stage
    // st-1, whose buffer the next load refills), load block st + NS - 1, compute block st.  Every stage loads
    // one set (the last block again once the blocks run out), so the waits stay uniform.  The buffer index
    // is a run-time value (one loop body for all stages).
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) issue(min(i, nsteps - 1), ring[i]);
    int cur = 0;
    for (int st = 0; st < nsteps; ++st) {
        const int fill = cur == 0 ? NS - 1 : cur - 1;
        // loads per stage: KL + 2 for the k'-loading waves, 2 for the others
        if (wave < KW) wait_vmcnt<(NS - 2) * (KL + 2)>();
        else wait_vmcnt<(NS - 2) * 2>();
        __builtin_amdgcn_s_barrier();
        issue(min(st + NS - 1, nsteps - 1), ring[fill]);
        compute(ring[cur]);
        cur = cur == NS - 1 ? 0 : cur + 1;
    }
    wait_vmcnt<0>();

    // ---- epilogue: dq = R^T dQ^T / sqrt(192) for this lane's query.  The tile leaves through the idle ring:
    // every wave puts its head's 32 rows there (row c NH + wave, 16-byte chunks XOR-swizzled by query within
    // groups of eight), then each store instruction writes whole runs of the NH heads of a query.
    const int qt = q0 + c;
    const float2 *qcs = a.rope + (size_t)min(max(qt - seq_start, 0), a.rope_len - 1) * NHALF;
    rope_back(dq[0], dq[1], qcs, hh);
    constexpr int RING = NS * (int)sizeof(DsqTile<NH>), ROWS = 32 * KCH * 16;   // bytes of one head's tile
    constexpr int ER = NH * ROWS <= RING ? 1 : (NH / 2) * ROWS <= RING ? 2 : 4, NHR = NH / ER;
    static_assert(NH % ER == 0 && NHR * ROWS <= RING, "dq staging");
    uint4 *stg = (uint4 *)ring;
    const int h0 = kvh * G + hg * NH;
#pragma unroll
    for (int rd = 0; rd < ER; ++rd) {
    __syncthreads();                        // every wave is done reading the ring
    if (wave / NHR == rd) {
        u16 *row = (u16 *)(stg + (c * NHR + wave % NHR) * KCH) + 4 * hh;
#pragma unroll
        for (int i = 0; i < 6; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = f2bf(dq[i][4 * jj + t] * RSQRT_DQK);
                const int k = 4 * i + jj;
                *(uint2 *)(row + 8 * ((k & ~7) | ((k & 7) ^ (c & 7)))) = __builtin_bit_cast(uint2, w);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 32 * NHR * KCH / (64 * NH); ++j) {
        const int g = 64 * NH * j + tid, R = g / KCH, k = g % KCH, qc = R / NHR, w = R % NHR;
        const uint4 x = stg[R * KCH + ((k & ~7) | ((k & 7) ^ (qc & 7)))];
        if (q0 + qc >= seq_start && q0 + qc < seq_end)
            st16u_nt(A.dq + ((size_t)(q0 + qc) * a.hq + h0 + rd * NHR + w) * DQK + 8 * k, x);
    }
    }
}

template <int GP>
hipError_t launch_dq(const BwdArgs &A, hipStream_t stream)
{
    const LayerArgs &a = A.L;
    const int G = a.hq / a.hkv;
    const bool win = a.window >= 0;
    // 4 waves (one per SIMD): the dq accumulators, q'/dO operands and scores need more than the 256
    // registers a wave may hold at two waves per SIMD
    constexpr int NW = 4;
    const int TT = 32 * NW / GP;
    const long tiles = (long)(a.T + TT - 1) / TT + a.batch;
    const long grid = tiles * (G / GP) * a.hkv;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    trace_begin(win ? "bwd_dq_swa" : "bwd_dq_global", stream);
    if (win) bwd_dq_kernel<NW, GP, true><<<(unsigned)grid, 64 * NW, 0, stream>>>(A);
    else bwd_dq_kernel<NW, GP, false><<<(unsigned)grid, 64 * NW, 0, stream>>>(A);
    trace_end(stream);
    return hipGetLastError();
}

template <int D, bool ROPE>
hipError_t launch_row_prep(const u16 *x, int H, u16 *rm, u16 *tr, const LayerArgs &a, int T_pad, hipStream_t stream)
{
    const long grid = (long)((T_pad + 63) / 64) * H;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    row_prep_kernel<D, ROPE><<<(unsigned)grid, 256, 0, stream>>>(x, H, rm, tr, a, T_pad);
    return hipGetLastError();
}

size_t al(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

bool bwd_group_supported(int group) { return group >= 1; }

hipError_t launch_zero_f32(float *p, int n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    zero_kernel<<<(n + 255) / 256, 256, 0, stream>>>(p, n);
    return hipGetLastError();
}

// workspace: lse2 and D [hq, T_pad] fp32, q' [T_pad, hq, 192], k' [T_pad, hkv, 192], k'^T [hkv, 192, T_pad]
// (bf16), dk|dv partials when splits > 1, and for the stored-dS path the block index and the dS blocks; each
// part 256-byte aligned
// Causal layers with large groups split each key tile's query heads over several workgroups, so that the
// first key tiles of a long sequence (which every later query sees) do not set the kernel's length alone:
// two splits where the 128-key tiles of all KV heads number 1024 or more (2048 workgroups, eight per CU),
// else four where the group allows (the per-GPU shapes of a head split: one or two KV heads).
static int dkv_splits(int T, int hq, int hkv, int window)
{
    const int G = hq / hkv;
    if (window >= 0 || G % 2 || G < 4) return 1;
    const long tiles = ((long)T + NKB - 1) / NKB * hkv;
    return tiles >= 1024 || G % 4 ? 2 : 4;
}

size_t bwd_workspace_bytes(int T, int hq, int hkv, int window)
{
    const size_t tp = (size_t)prep_tpad(T);
    const int sp = dkv_splits(T, hq, hkv, window);
    return 2 * al(tp * hq * 4) + al(tp * hq * DQK * 2) + al(tp * hkv * DQK * 2) + al(tp * hkv * DQK * 2) +
           (sp > 1 ? al((size_t)sp * tp * hkv * (DQK + DVV) * 4) : 0);
}

// Stored-dS path: an upper bound on the dS blocks of one head, from the total tokens T, the number of
// sequences and the longest one.  A sequence of L tokens has nq <= L / 32 + 1.44 query tiles; causal rows
// hold nq (nq + 1) / 2 blocks (sum of L^2 <= T max_seqlen), sliding-window rows nq row-width blocks.
static int64_t ds_blocks_bound(int T, int window, int batch, int max_seqlen)
{
    const int64_t t32 = (int64_t)T / 32 + 1;
    if (window >= 0) return (t32 + 2 * (int64_t)batch + 1) * ds_row_width(window);
    return ((int64_t)T * max_seqlen / 1024 + 4 * t32 + 4 * (int64_t)batch) / 2 + (int64_t)batch + 1;
}

// Only where the dQ kernel of the stored-dS path applies: query heads in groups of four per KV head.
size_t bwd_workspace_bytes_ds(int T, int hq, int hkv, int window, int batch, int max_seqlen)
{
    if (hq % hkv || (hq / hkv) % 4 || T <= 0) return 0;
    const int64_t blocks = ds_blocks_bound(T, window, batch, max_seqlen);
    return bwd_workspace_bytes(T, hq, hkv, window) + al((size_t)(batch + 1) * 8) + al((size_t)hq * blocks * 2048);
}

void bwd_carve(void *ws, int T, int hq, int hkv, BwdArgs *A, bool stored_ds, int batch, int max_seqlen)
{
    const size_t tp = (size_t)prep_tpad(T);
    char *p = (char *)ws;
    A->T_pad = (int)tp;
    A->lse2 = (float *)p;
    p += al(tp * hq * 4);
    A->delta = (float *)p;
    p += al(tp * hq * 4);
    A->W.qr = (u16 *)p;
    p += al(tp * hq * DQK * 2);
    A->W.kr = (u16 *)p;
    p += al(tp * hkv * DQK * 2);
    A->W.krt = (u16 *)p;
    p += al(tp * hkv * DQK * 2);
    A->splits = dkv_splits(T, hq, hkv, A->L.window);
    A->dkv_part = A->splits > 1 ? (float *)p : nullptr;
    if (A->splits > 1) p += al((size_t)A->splits * tp * hkv * (DQK + DVV) * 4);
    A->ds = nullptr;
    A->ds_index = nullptr;
    if (stored_ds) {
        A->ds_index = (int64_t *)p;
        p += al((size_t)(batch + 1) * 8);
        A->ds = (u16 *)p;
        (void)max_seqlen;
    }
}

hipError_t launch_bwd(const BwdArgs &A, hipStream_t stream)
{
    const LayerArgs &a = A.L;
    const dim3 pre_grid((unsigned)(A.T_pad / 16), (unsigned)((a.hq + 15) / 16));   // T_pad is a multiple of 16
    if (pre_grid.y > 65535) return hipErrorInvalidConfiguration;
    trace_begin(a.window >= 0 ? "bwd_pre_swa" : "bwd_pre_global", stream);
    bwd_pre_kernel<<<pre_grid, 256, 0, stream>>>(A);
    trace_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (A.dsink) {
        trace_begin(a.window >= 0 ? "bwd_dsink_swa" : "bwd_dsink_global", stream);
        bwd_dsink_kernel<<<a.hq, 1024, 0, stream>>>(A);
        trace_end(stream);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!A.qr_given) {
        trace_begin(a.window >= 0 ? "bwd_prep_q_swa" : "bwd_prep_q_global", stream);
        e = launch_row_prep<DQK, true>(a.q, a.hq, A.W.qr, nullptr, a, A.T_pad, stream);
        trace_end(stream);
        if (e != hipSuccess) return e;
    }
    if (!A.kr_given) {
        trace_begin(a.window >= 0 ? "bwd_prep_k_swa" : "bwd_prep_k_global", stream);
        // the transposed k' copy serves only the dQ kernel that recomputes S and dP (least workspace)
        e = launch_row_prep<DQK, true>(a.k, a.hkv, A.W.kr, A.ds ? nullptr : A.W.krt, a, A.T_pad, stream);
        trace_end(stream);
        if (e != hipSuccess) return e;
    }

    if (A.ds) {
        trace_begin(a.window >= 0 ? "bwd_ds_index_swa" : "bwd_ds_index_global", stream);
        bwd_ds_index_kernel<<<1, 256, 0, stream>>>(A);
        trace_end(stream);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long kv_tiles = (long)(a.T + NKB - 1) / NKB + a.batch;
    const long kv_grid = kv_tiles * a.hkv * A.splits;
    if (kv_grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    trace_begin(a.window >= 0 ? "bwd_dkdv_swa" : "bwd_dkdv_global", stream);
    if (a.window >= 0) bwd_dkdv_kernel<true><<<(unsigned)kv_grid, 512, 0, stream>>>(A);
    else bwd_dkdv_kernel<false><<<(unsigned)kv_grid, 512, 0, stream>>>(A);
    trace_end(stream);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (A.splits > 1) {
        const long items = (long)a.T * a.hkv * 40;
        trace_begin(a.window >= 0 ? "bwd_dkv_reduce_swa" : "bwd_dkv_reduce_global", stream);
        bwd_dkv_reduce_kernel<<<(unsigned)((items + 255) / 256), 256, 0, stream>>>(A);
        trace_end(stream);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int G = a.hq / a.hkv;
    if (A.ds) {
        const int nh = G % 16 == 0 && a.window < 0 ? 16 : G % 8 == 0 ? 8 : 4;
        const long grid = ((long)a.T / 32 + 2L * a.batch) * (G / nh) * a.hkv;
        if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
        trace_begin(a.window >= 0 ? "bwd_dq_ds_swa" : "bwd_dq_ds_global", stream);
        if (a.window >= 0 && nh == 8) bwd_dq_ds_kernel<8, true, 2, 2><<<(unsigned)grid, 512, 0, stream>>>(A);
        else if (a.window >= 0) bwd_dq_ds_kernel<4, true, 3, 2><<<(unsigned)grid, 256, 0, stream>>>(A);
        else if (nh == 16) bwd_dq_ds_kernel<16, false, 3, 1><<<(unsigned)grid, 1024, 0, stream>>>(A);
        else if (nh == 8) bwd_dq_ds_kernel<8, false, 5, 1><<<(unsigned)grid, 512, 0, stream>>>(A);
        else bwd_dq_ds_kernel<4, false, 5, 1><<<(unsigned)grid, 256, 0, stream>>>(A);
        trace_end(stream);
        return hipGetLastError();
    }
    if (G % 8 == 0) return launch_dq<8>(A, stream);
    if (G % 4 == 0) return launch_dq<4>(A, stream);
    if (G % 2 == 0) return launch_dq<2>(A, stream);
    return launch_dq<1>(A, stream);
}

}  // namespace mimo
