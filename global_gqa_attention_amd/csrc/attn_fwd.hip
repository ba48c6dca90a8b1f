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
//   * A prep kernel (attn_prep.hip) first writes RoPE-rotated K and per-head transposed V into the
//     workspace.  The hot loop then moves K and V^T tiles from HBM straight into LDS with
//     global_load_lds_dwordx4 (no register staging, no per-tile arithmetic), double-buffered: the next tile
//     is in flight while the current one is computed, ordered by one explicit vmcnt wait and plain
//     s_barriers.  The 16-byte chunks of each LDS row are XOR-swizzled by row (the per-lane source
//     addresses are permuted), so every MFMA operand read is free of bank conflicts.
//   * Each wave owns 32 query rows; a workgroup of NW waves owns 32 NW rows: TT = 32 NW / GP consecutive
//     tokens x GP query heads of one KV group, so all GP heads reuse every K/V tile.  Causal layers use 12
//     waves (three per SIMD, one K/V stream for 384 rows), sliding-window layers 4 waves (a short key span:
//     the tile's tokens plus 128 keys back).  32-key blocks that no row of a wave can see are skipped.
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: the query is the MFMA column, so each lane owns a query
//     (lanes l and l ^ 32 split its keys); row max and row sum need one permlane32 swap, and the rescale of
//     the output accumulator is per lane.  O^T = V^T . P^T takes the score registers as its B operand, with
//     V^T's 4-key chunks stored in the order the score registers hold the keys.  Q is rotated once in
//     registers (cos/sin from a table built in fp64).
//   * Per 32-key block a wave reads all 12 K operands before its S MFMAs, and the 8 V^T operands right
//     after them, so the V reads land while the softmax runs; the other wave on the SIMD fills the matrix
//     pipe meanwhile.
//   * Online softmax in base 2: p = exp2(s * scale - m) is one fma and one v_exp; probabilities are packed
//     to bf16 in pairs and the row sum adds exactly those packed values (v_dot2 with ones), so numerator
//     and denominator agree.  The sink starts the running max and sum.  The reference max moves only when
//     a block's max exceeds it by 2^8, so most blocks skip the rescale of the accumulator (exact either
//     way: numerator and denominator share the reference); the branch is wave-uniform.  Only blocks that
//     cross a causal, window or sequence boundary evaluate the mask (one wave-uniform branch per block).
#include "device_common.hpp"
#include "internal.hpp"

namespace mimo {
namespace {

constexpr int KCH = DQK / 8;   // 16-byte chunks per K row (24)
constexpr float RESCALE_TH = 8.f;   // keep a stale running max until the true one exceeds it by 2^8
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// K tile in LDS: row r (key), 24 chunks of 16 B (384-byte rows); V^T tile: row d (dim), BN / 8 chunks
// (128-byte rows for 64-key tiles, 64-byte rows for 32-key tiles).
__device__ __forceinline__ int kpos(int r, int q) { return swz384(r, q); }
template <int BN>
__device__ __forceinline__ int vpos(int d, int q) { return BN == 64 ? swz128(d, q) : swz64(d, q); }

// NW waves per workgroup (32 query rows each) share one stream of BN-key K/V tiles.  Causal layers: 12
// waves, one workgroup per CU, so three waves share each SIMD and one's softmax and LDS waits overlap the
// others' MFMAs; that leaves 168 registers per wave: K operands are read four at a time (KA = 4) and the
// tiles hold 32 keys in a 3-stage ring (60 KB: 64-key tiles would put ring buffers beyond the 64 KB reach of
// an LDS instruction's offset field, which costs address registers this wave cannot spare).  Sliding-window
// layers: 4 waves, 32-key tiles double-buffered (40 KB) and KA = 4 so that three workgroups fit on a CU (OCC):
// these short work items wait mostly on HBM (Q and the first tiles), and more resident workgroups keep more
// loads in flight.  q passes through LDS first in both forms: a lane that loads its own row touches 32 rows
// per load instruction, while the copy into LDS reads whole runs of rows per instruction; the rotated q for
// the backward leaves the same way.  Sliding window: 48 KB at the start of the pool, the first tile issued
// after it.  Causal: 144 KB behind the first K tile (156 KB of the CU's 160 KB), that tile's V^T issued once
// every wave has read its q.  After the key loop, O leaves through LDS in both forms.
template <int NW, int GP, bool SINK, bool WIN, int BN, int KA, int OCC>
__global__ __launch_bounds__(64 * NW, OCC) void attn_fwd_kernel(const FwdArgs A)
{
    constexpr int VCH = BN / 8;                // 16-byte chunks per V^T row
    constexpr int NT = 64 * NW;                // threads per workgroup
    constexpr int BM = 32 * NW;                // query rows per workgroup
    constexpr int KLOADS = BN * KCH / NT;      // global_load_lds per thread per K tile
    constexpr int VLOADS = DVV * VCH / NT;     // ... per V^T tile (every thread)
    constexpr int VEXTRA = DVV * VCH - VLOADS * NT;   // V^T chunks left over: one more for threads below this
    static_assert(KLOADS * NT == BN * KCH && VEXTRA % 64 == 0, "tile split");
    const LayerArgs &a = A.L;
    constexpr int NBUF = NW >= 8 ? 3 : 2;      // LDS stages: three where one workgroup owns the CU
    constexpr int KS = BN * KCH, VS = DVV * VCH;                 // 16-byte chunks of a K and a V^T tile
    // the workgroup's q rows pass through LDS first: sliding window from the start of the pool (the first
    // tile is issued after them), causal behind the first K tile (in flight meanwhile; its V^T comes after)
    constexpr int QOFF = WIN ? 0 : KS, QEND = QOFF + BM * KCH;
    constexpr int OSTAGE = BM * DVV / 8;                          // the epilogue's O rows (16-byte chunks)
    constexpr int POOL0 = NBUF * (KS + VS) > QEND ? NBUF * (KS + VS) : QEND;
    constexpr int POOL = POOL0 > OSTAGE ? POOL0 : OSTAGE;
    __shared__ __attribute__((aligned(16))) uint4 lds[POOL];
    uint4 *const sK0 = lds, *const sV0 = lds + KS, *const sK1 = lds + KS + VS, *const sV1 = lds + 2 * KS + VS;
    uint4 *const sK2 = lds + 2 * (KS + VS), *const sV2 = lds + 3 * KS + 2 * VS;   // NBUF == 3 only

    constexpr int TT = BM / GP;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) by construction
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
    // token tiles counted from the last tile of the last sequence
    const SeqPos sp = seq_lookup_rev(a.cu, a.batch, tile, [](int s, int e) { return (e - s + TT - 1) / TT; });
    if (sp.b < 0) return;
    const int seq_start = sp.start, seq_end = sp.end;
    const int tr = (seq_end - seq_start + TT - 1) / TT - 1 - sp.j;
    const int t0 = seq_start + tr * TT;
    const int t_last = min(t0 + TT - 1, seq_end - 1);
    const int h0 = kvh * G + hgi * GP;
    // key stream of the sequence: its first key is kseq, query token t sits at key index t + kofs and at
    // RoPE position t + pofs (without a cache: the tokens themselves, positions from the sequence start)
    int kofs = 0, kseq = seq_start, pofs = -seq_start;
    if (A.C.cu_cache) {
        const int c0 = A.C.cu_cache[sp.b], c1 = A.C.cu_cache[sp.b + 1];
        kofs = c1;
        kseq = c0 + seq_start;
        pofs = A.C.positions[sp.b] - seq_start;
    }

    // ---- key range: tiles start on a 16-key boundary (the V^T chunk order is per 16 keys); keys of a
    // previous sequence that this brings in are masked
    // The prepared key stream has T_pad rows (a multiple of 16) and every tile read must stay inside it: the
    // first tile starts at most at T_pad - BN, the last ends at most at row T_pad - 1, and a range that
    // holds no tile gives no key step at all (these bounds bind only when the cache index arrays claim more
    // rows than the sizes given; the rows are then wrong, but nothing outside the workspace is read).
    const int klo = WIN ? max(kseq, t0 + kofs - a.window) : kseq;
    const int kstart = min(max(klo, 0) & ~15, A.P.T_pad - BN);
    const int khi = min(t_last + kofs, A.P.T_pad - BN - 1);
    const int nkt = max((khi - kstart + BN) / BN, 0);

    // ---- direct HBM -> LDS loads of one K tile and one V^T tile (slot s = NT j + tid of each array): the
    // per-lane byte offsets are fixed, the tile start is a wave-uniform base
    const u16 *kr_base = A.P.kr + (size_t)kvh * DQK;
    const size_t kr_row = (size_t)a.hkv * DQK;
    const u16 *vt_base = A.P.vt + (size_t)kvh * DVV * A.P.T_pad;
    uint32_t koff[KLOADS], voff[VLOADS > 0 ? VLOADS : 1];
#pragma unroll
    for (int j = 0; j < KLOADS; ++j) {
        const int slot = NT * j + tid, r = slot / KCH, p = slot % KCH;
        koff[j] = (uint32_t)((r * kr_row + 8 * kpos(r, p)) * 2);    // kpos is an involution
    }
#pragma unroll
    for (int j = 0; j < VLOADS; ++j) {
        const int slot = NT * j + tid, d = slot / VCH, p = slot % VCH;
        voff[j] = (uint32_t)(((size_t)d * A.P.T_pad + 8 * vpos<BN>(d, p)) * 2);
    }
    uint32_t vextra = 0;
    if constexpr (VEXTRA > 0) {
        const int slot = NT * VLOADS + min(tid, VEXTRA - 1), d = slot / VCH, p = slot % VCH;
        vextra = (uint32_t)(((size_t)d * A.P.T_pad + 8 * vpos<BN>(d, p)) * 2);
    }
    auto issue_tile = [&](int k0, uint4 *sk, uint4 *sv) {
        const u16 *kb = kr_base + (size_t)k0 * kr_row;
        const u16 *vb = vt_base + k0;
#pragma unroll
        for (int j = 0; j < KLOADS; ++j) lds_dma16(kb, koff[j], sk + NT * j + 64 * wave);
#pragma unroll
        for (int j = 0; j < VLOADS; ++j) lds_dma16(vb, voff[j], sv + NT * j + 64 * wave);
        if constexpr (VEXTRA > 0) {
            if (wave < VEXTRA / 64) lds_dma16(vb, vextra, sv + NT * VLOADS + 64 * wave);
        }
    };
    // this wave's loads of one tile (waves below VEXTRA / 64 issue one more V^T chunk)
    auto wait_tile = [&]() {
        if constexpr (VEXTRA > 0) {
            if (wave < VEXTRA / 64) wait_vmcnt<KLOADS + VLOADS + 1>();
            else wait_vmcnt<KLOADS + VLOADS>();
        } else {
            wait_vmcnt<KLOADS + VLOADS>();
        }
    };
    auto issue_v = [&](int k0, uint4 *sv) {
        const u16 *vb = vt_base + k0;
#pragma unroll
        for (int j = 0; j < VLOADS; ++j) lds_dma16(vb, voff[j], sv + NT * j + 64 * wave);
        if constexpr (VEXTRA > 0) {
            if (wave < VEXTRA / 64) lds_dma16(vb, vextra, sv + NT * VLOADS + 64 * wave);
        }
    };
    if constexpr (!WIN) {
        const u16 *kb = kr_base + (size_t)kstart * kr_row;
#pragma unroll
        for (int j = 0; j < KLOADS; ++j) lds_dma16(kb, koff[j], sK0 + NT * j + 64 * wave);
    }

    // ---- this lane's query row, rotated in registers
    const int r = wave * 32 + c;
    const int qt = t0 + r / GP;
    const int qh = h0 + r % GP;
    const bool qvalid = qt < seq_end;
    bf16x8 qf[12];
    {
        const int qtl = qvalid ? qt : t_last;
        const float2 *cs = a.rope + (size_t)min(max(qtl + pofs, 0), a.rope_len - 1) * NHALF + 8 * hh;
        float2 c0[8], c1[8];
        // the wave's 32 rows (768 16-byte chunks, GP-row runs contiguous in memory) are copied into LDS by
        // whole runs, chunk slot g by instruction g / 64, swizzled like a K tile; each lane then reads its
        // own row and rotates it.  The rotated q for the backward leaves the same way: the rotated chunks go
        // back into their slots and each instruction stores whole runs.  Once every wave is done with its
        // q, the loads that this LDS waited for are issued (sliding window: the first tile; causal: the
        // first tile's V^T, then the second tile).
        const u16 *qbase = a.q + ((size_t)t0 * a.hq + h0) * DQK;
        uint4 *qs = lds + QOFF + 32 * KCH * wave;
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            const int g = 64 * i + lane, rw = g / KCH, rr = wave * 32 + rw;
            const int tk = min(rr / GP, t_last - t0);
            lds_dma16_nt(qbase, (uint32_t)(((tk * a.hq + rr % GP) * DQK + 8 * kpos(rw, g % KCH)) * 2), qs + 64 * i);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            c0[t] = cs[t];
            c1[t] = cs[16 + t];
        }
        wait_vmcnt<0>();
#pragma unroll
        for (int s = 0; s < 12; ++s) qf[s] = __builtin_bit_cast(bf16x8, qs[KCH * c + kpos(c, 2 * s + hh)]);
        rope_pair(qf[0], qf[2], c0);
        rope_pair(qf[1], qf[3], c1);
        if (A.q_rot) {
#pragma unroll
            for (int s = 0; s < 4; ++s) qs[KCH * c + kpos(c, 2 * s + hh)] = __builtin_bit_cast(uint4, qf[s]);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own slots, read by its lanes
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                const int g = 64 * i + lane, rw = g / KCH, rr = wave * 32 + rw;
                const int tok = t0 + rr / GP;
                const uint4 x = qs[g];
                if (tok < seq_end)
                    st16u_nt(A.q_rot + ((size_t)tok * a.hq + h0 + rr % GP) * DQK + 8 * kpos(rw, g % KCH), x);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        if constexpr (WIN) issue_tile(kstart, sK0, sV0);
        else issue_v(kstart, sV0);
    }

    // this wave's rows sit at key indices [wt0, wt1]; 32-key blocks outside [wklo, wkhi] are skipped
    const int wt0 = t0 + (wave * 32) / GP + kofs;
    const int wt1 = min(t0 + (wave * 32 + 31) / GP, seq_end - 1) + kofs;
    const int wklo = WIN ? max(kseq, wt0 - a.window) : kseq;
    const int wkhi = wt1;

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

    // ---- one tile: S^T = K Q^T, online softmax, O^T += V^T P^T (two 32-key blocks).  The V^T operands of a
    // block are read before its softmax, so they land while the softmax runs.
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
    const int qk = qt + kofs;   // this row's key index
    const uint32_t ub = (uint32_t)(WIN ? min(a.window, qk - kseq) : qk - kseq);
    auto compute_tile = [&](int k0, const uint4 *skb, const uint4 *svb) {
        const u16 *kt = (const u16 *)skb;
        const u16 *vtt = (const u16 *)svb;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            const int kbase = k0 + 32 * kb;
            if (kbase > wkhi || kbase + 31 < wklo) continue;     // no row of this wave sees these 32 keys
            const int kr_ = 32 * kb + c;
            bf16x8 kop[KA];
#pragma unroll
            for (int s = 0; s < KA; ++s) kop[s] = ld16(kt + (kr_ * KCH + kpos(kr_, 2 * s + hh)) * 8);
            f32x16 sacc = f32x16{};
#pragma unroll
            for (int s = 0; s < 12; ++s) {
                sacc = mfma32(kop[s % KA], qf[s], sacc);
                if (s + KA < 12) kop[s % KA] = ld16(kt + (kr_ * KCH + kpos(kr_, 2 * (s + KA) + hh)) * 8);
            }
            // V^T operand m = 2 i + s (rows 32 i + c, k-step s); KA == 12: all eight read before the softmax,
            // else the first two before it (they land while the softmax runs) and the rest two ahead of the
            // P V MFMAs (fewer registers)
            auto vread = [&](int m) {
                const int d = 32 * (m >> 1) + c;
                return ld16(vtt + (d * VCH + vpos<BN>(d, 4 * kb + 2 * (m & 1) + hh)) * 8);
            };
            constexpr int VA = KA == 12 ? 8 : 2;
            bf16x8 vop[VA];
#pragma unroll
            for (int m = 0; m < VA; ++m) vop[m] = vread(m);
            __builtin_amdgcn_sched_barrier(0);
            float sv[16];
            float mxa = -INFINITY, mxb = -INFINITY;
            const bool need_mask = (kbase + 31 > wt0) || (kbase < kseq) || (WIN && kbase < wt1 - a.window);
            if (need_mask) {
                const int dlt = qk - (kbase + 4 * hh);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int cj = 8 * (j >> 2) + (j & 3);
                    sv[j] = (uint32_t)(dlt - cj) <= ub ? sacc[j] : -INFINITY;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) sv[j] = sacc[j];
            }
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                mxa = fmaxf(mxa, sv[j]);
                mxb = fmaxf(mxb, sv[j + 1]);
            }
            const float mx = pair_max(fmaxf(mxa, mxb)) * a.scale_log2;
            // lazy rescale: move the reference max only when the block max exceeds it by 2^8; the branch is
            // wave-uniform so the accumulators are touched only when some row needs it
            const bool grow = mx > m_run + RESCALE_TH;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                const float alpha = grow ? fast_exp2(m_run - mx) : 1.f;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] *= alpha;
                m_run = grow ? mx : m_run;
            }
            const float nref = m_run == -INFINITY ? 0.f : -m_run;
            uint32_t pw[8];
            float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const float p0 = fast_exp2(__builtin_fmaf(sv[2 * w], a.scale_log2, nref));
                const float p1 = fast_exp2(__builtin_fmaf(sv[2 * w + 1], a.scale_log2, nref));
                pw[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, bf16x2));
                if (w & 1) ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[w]), ones, ps1, false);
                else ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[w]), ones, ps0, false);
            }
            l_run += ps0 + ps1;
            const bf16x8 pf[2] = {__builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3])),
                                  __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]))};
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                o[m >> 1] = mfma32(vop[m % VA], pf[m & 1], o[m >> 1]);
                if (VA < 8 && m + VA < 8) vop[m % VA] = vread(m + VA);
            }
        }
    };

    const int klast = kstart + max(nkt - 1, 0) * BN;   // first row of the last tile (kstart when there is none)
    if constexpr (NBUF == 3) {
        // ---- three-stage ring, unrolled by three so each step names its buffers.  Every step issues
        // exactly one tile (the last valid tile again once the range is exhausted), so the loads in flight
        // are always the current tile and the next one: waiting for all but the newest tile's loads makes
        // the current tile land.  The barrier after that wait also tells this wave that every wave has
        // finished the previous step, whose buffer the new loads then refill.  The LDS tiles are written
        // only by these direct loads, so a plain s_barrier suffices.
        issue_tile(min(kstart + BN, klast), sK1, sV1);
        auto step = [&](int it, const uint4 *ck, const uint4 *cv, uint4 *nk, uint4 *nv) {
            wait_tile();
            __builtin_amdgcn_s_barrier();
            issue_tile(min(kstart + (it + 2) * BN, klast), nk, nv);
            if (it < nkt) compute_tile(kstart + it * BN, ck, cv);
        };
        for (int it = 0; it < nkt; it += 3) {
            step(it, sK0, sV0, sK2, sV2);
            step(it + 1, sK1, sV1, sK0, sV0);
            step(it + 2, sK2, sV2, sK1, sV1);
        }
    } else {
        // ---- double-buffered loop, unrolled by two so each half names its own buffers.  Every half
        // issues exactly one tile (the last valid tile again once the range is exhausted), so the number
        // of loads in flight is the same on every path: the wait for a buffer is always "all but the
        // newest tile's loads".  Each wave waits (vmcnt) for its own loads of the tile it reads next, and
        // reaches the following barrier only after its MFMAs consumed every LDS read of the buffer that
        // is refilled next.
        for (int it = 0; it < nkt; it += 2) {
            const int k0 = kstart + it * BN;
            issue_tile(min(k0 + BN, klast), sK1, sV1);
            wait_tile();
            __builtin_amdgcn_s_barrier();       // tile it is in buffer 0 for every wave
            compute_tile(k0, sK0, sV0);
            __builtin_amdgcn_s_barrier();       // every wave is done reading buffer 0
            issue_tile(min(k0 + 2 * BN, klast), sK0, sV0);
            wait_tile();
            __builtin_amdgcn_s_barrier();       // tile it+1 is in buffer 1 for every wave
            if (it + 1 < nkt) compute_tile(k0 + BN, sK1, sV1);
            __builtin_amdgcn_s_barrier();       // every wave is done reading buffer 1
        }
    }
    wait_vmcnt<0>();                        // no load may still target this workgroup's LDS at exit

    // ---- epilogue: out = 0.707 * O / l, LSE = ln(l) + max.  O leaves through the idle K/V ring: each lane
    // puts its row there (16-byte chunks XOR-swizzled by row), then every store instruction writes whole
    // runs of rows instead of touching 32 rows.
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? VSCALE / l_tot : 0.f;   // no visible key and no sink: zero output
    if (qvalid && A.lse && hh == 0) A.lse[(size_t)qh * a.T + qt] = (m_run + __log2f(l_tot)) * LN2;
    __builtin_amdgcn_s_barrier();           // every wave is done reading the ring
    {
        // the lane index again from mbcnt: cheaper to recompute here than to keep across the key loop
        const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        const int lc = ln & 31, lh = ln >> 5;
        u16 *orow = (u16 *)lds + (size_t)(wave * 32 + lc) * DVV + 4 * lh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = f2bf(o[i][4 * jj + t] * inv);
                *(uint2 *)(orow + 8 * ((4 * i + jj) ^ (lc & 15))) = __builtin_bit_cast(uint2, w);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own rows, read by its lanes
        const uint4 *ws = lds + wave * 32 * (DVV / 8);
        u16 *obase = A.out + ((size_t)t0 * a.hq + h0) * DVV;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int g = 64 * j + ln, rw = g >> 4, p = g & 15, r = wave * 32 + rw;
            const uint4 x = ws[16 * rw + (p ^ (rw & 15))];
            if (t0 + r / GP < seq_end) st16u_nt(obase + (uint32_t)(((r / GP) * a.hq + r % GP) * DVV + 8 * p), x);
        }
    }
}

template <int GP>
hipError_t launch_gp(const FwdArgs &A, hipStream_t stream)
{
    const LayerArgs &a = A.L;
    const int G = a.hq / a.hkv;
    const bool sink = a.sink != nullptr, win = a.window >= 0;
    const int NW = win ? 4 : 12;
    const int TT = 32 * NW / GP;
    // upper bound on the number of token tiles: sum ceil(len/TT) <= ceil(T/TT) + batch
    const long tiles = (long)(a.T + TT - 1) / TT + a.batch;
    const long grid = tiles * (G / GP) * a.hkv;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    trace_begin(win ? "attn_fwd_swa" : "attn_fwd_global", stream);
    if (sink && win) attn_fwd_kernel<4, GP, true, true, 32, 4, 3><<<(unsigned)grid, 256, 0, stream>>>(A);
    else if (win) attn_fwd_kernel<4, GP, false, true, 32, 4, 3><<<(unsigned)grid, 256, 0, stream>>>(A);
    else if (sink) attn_fwd_kernel<12, GP, true, false, 32, 4, 1><<<(unsigned)grid, 768, 0, stream>>>(A);
    else attn_fwd_kernel<12, GP, false, false, 32, 4, 1><<<(unsigned)grid, 768, 0, stream>>>(A);
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
    hipError_t e = A.C.cu_cache ? launch_kv_prep_cached(a, A.P, A.C, stream) : launch_kv_prep(a, A.P, stream);
    if (e != hipSuccess) return e;
    const int G = a.hq / a.hkv;
    // pack up to 8 heads of a group: 32 tokens x 8 heads per workgroup for sliding-window layers (short key
    // span), and the same for causal layers (each K/V tile serves 8 heads; little waste on the diagonal).
    if (G % 8 == 0) return launch_gp<8>(A, stream);
    if (G % 4 == 0) return launch_gp<4>(A, stream);
    if (G % 2 == 0) return launch_gp<2>(A, stream);
    return launch_gp<1>(A, stream);
}

size_t fwd_workspace_bytes(int T, int hq, int hkv, int window)
{
    (void)hq;
    (void)window;
    return prep_bytes(T, hkv);
}

hipError_t launch_rope_table(float2 *table, int npos, double base, hipStream_t stream)
{
    const long n = (long)npos * NHALF;
    const long blocks = (n + 255) / 256;
    rope_table_kernel<<<(unsigned)blocks, 256, 0, stream>>>(table, npos, base);
    return hipGetLastError();
}

}  // namespace mimo
