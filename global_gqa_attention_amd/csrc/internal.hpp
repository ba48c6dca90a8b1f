// internal.hpp -- argument blocks and launchers shared between the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mimo {

// One prefill layer (forward or backward).  All pointers are device pointers.
struct LayerArgs {
    const uint16_t *q, *k, *v;     // bf16 [T,hq,192], [T,hkv,192], [T,hkv,128]
    const float *sink;             // [hq] or nullptr
    const int32_t *cu;             // [batch+1]
    const float2 *rope;            // (cos, sin) [rope_len, 32]
    int batch, T, window, hq, hkv, rope_len;
    float scale_log2;              // log2(e) / sqrt(192)
};

// Prepared K/V in the workspace (written by kv_prep, read by the hot loops through global_load_lds).
struct KVPrep {
    uint16_t *kr;                  // bf16 [T_pad, hkv, 192]: K with RoPE applied
    uint16_t *vt;                  // bf16 [hkv, 128, T_pad]: V transposed, 4-token chunks permuted
    uint16_t *k_rot;               // bf16 [T, hkv, 192]: a copy of kr's first T rows for the caller, or nullptr
    int T_pad;                     // tokens rounded up to 16, plus 64 zero-filled
};
inline int prep_tpad(int T) { return (T + 15) / 16 * 16 + 64; }
// The direct-to-LDS copies address a tile with a 64-bit wave-uniform base plus a 32-bit per-lane byte offset.
// Transposed copies (dim-major, T_pad tokens per row) put the dim index into that offset: 128 rows of V^T in
// the forward, 192 rows of k'^T in the backward.  Key streams whose offsets would pass 2^32 are refused on
// the host.
inline bool fwd_stream_fits(long long rows)
{
    return rows >= 0 && rows <= 0x7fffff00LL && (long long)prep_tpad((int)rows) * 128 * 2 <= 0xffffffffLL;
}
inline bool bwd_stream_fits(long long rows)
{
    return rows >= 0 && rows <= 0x7fffff00LL && (long long)prep_tpad((int)rows) * 192 * 2 <= 0xffffffffLL;
}
size_t prep_bytes(int T, int hkv);
void prep_carve(void *ws, int T, int hkv, KVPrep *p);

// A cached prefix in front of the new tokens (prefill of a chunk against the KV cache).  Sequence b has
// cache rows cu_cache[b] .. cu_cache[b+1]-1: the keys just before its new tokens, in position order, with
// RoPE already applied to K and V unscaled; its first new token sits at positions[b].  The prep kernel
// lays the cache rows and the new tokens' keys out as one key stream per sequence (sequence b's keys start
// at cu_cache[b] + cu[b]), so the key index of new token t is t + cu_cache[b+1].
struct CacheArgs {
    const uint16_t *k_cache, *v_cache;   // bf16 [Tc,hkv,192] (rotated), [Tc,hkv,128]; paged: the pools
    const int32_t *cu_cache;             // [batch+1], or nullptr: no cache (plain prefill)
    const int32_t *page_table;           // paged cache: pool row of cache row i is page_table[i], or nullptr
    const int32_t *positions;            // [batch]
    int Tc;                              // cache rows in all
};

struct FwdArgs {
    LayerArgs L;
    KVPrep P;                      // keys of the cached prefix and the new tokens when C.cu_cache is set
    CacheArgs C;
    uint16_t *out;                 // bf16 [T,hq,128]
    float *lse;                    // fp32 [hq,T] or nullptr
    uint16_t *q_rot;               // bf16 [T,hq,192] rotated q, or nullptr
};

// DMA-ready copies the backward prepares in its workspace (see attn_bwd.hip).
struct BwdPrep {
    uint16_t *qr;                  // bf16 [T_pad, hq, 192]   q with RoPE applied
    uint16_t *kr;                  // bf16 [T_pad, hkv, 192]  k with RoPE applied
    uint16_t *krt;                 // bf16 [hkv, 192, T_pad]  the same, transposed
};

struct BwdArgs {
    LayerArgs L;
    BwdPrep W;
    const uint16_t *out, *dout;    // bf16 [T,hq,128]
    const float *lse;              // [hq,T]
    uint16_t *dq, *dk, *dv;        // bf16 outputs
    float *dsink;                  // [hq] or nullptr
    float *delta;                  // workspace: D = rowsum(dO * O) [hq,T_pad]
    float *lse2;                   // workspace: LSE * log2(e) [hq,T_pad]
    float *dkv_part;               // workspace: fp32 dk|dv partials [splits, T_pad, hkv, 320] (splits > 1)
    int T_pad;
    int qr_rows;                   // rows of W.qr that may be read: T_pad (prepared here) or T (the caller's)
    bool qr_given;                 // W.qr is the forward's q_rot: no prep pass for q
    int kr_rows;                   // rows of W.kr that may be read: T_pad (prepared here) or T (the caller's)
    bool kr_given;                 // W.kr is the forward's k_rot: no prep pass for k
    int splits;                    // query heads of a group are split over this many key-tile workgroups
    // stored-dS path (nullptr: dQ recomputes S and dP): the dK/dV kernel writes every 32 x 32 bf16 block of
    // dS it computes, the dQ kernel reads them back.  ds_index[b] = first block of sequence b within a head,
    // ds_index[batch] = blocks per head.
    uint16_t *ds;
    int64_t *ds_index;
    int64_t ds_cap;                // blocks that fit in the workspace (guards a max_seqlen below the truth)
};
void bwd_carve(void *ws, int T, int hq, int hkv, BwdArgs *A, bool stored_ds, int batch, int max_seqlen);

struct DecodeArgs {
    const uint16_t *q, *k_new, *v_new, *k_cache, *v_cache;   // paged: k_cache / v_cache are the pools
    const int32_t *cu_cache, *positions;
    const int32_t *page_table;     // paged cache: pool row of each cache row (cu_cache indexes it), or nullptr
    const float *sink;
    uint16_t *out;
    float *part_o;                 // workspace [batch, hq, splits, 128]
    float *part_ml;                // workspace [batch, hq, splits, 2] (max in log2 units, sum)
    int batch, window, hq, hkv, splits, split_len;
    int nq;                        // query tokens per sequence: 1 (decode, k_new given) or the draft count
                                   // (verify, k_new == nullptr: the drafts' keys are the last nq cache rows)
    double rope_base;
    float scale_log2;
};

// Tracing hooks (no-ops unless tracing is enabled): bracket one kernel launch on `stream`.
void trace_begin(const char *name, hipStream_t stream);
void trace_end(hipStream_t stream);

// Returns hipSuccess or the launch error.  Each launcher picks its kernel variant from the arguments.
hipError_t launch_kv_prep(const LayerArgs &a, const KVPrep &p, hipStream_t stream);
hipError_t launch_kv_prep_cached(const LayerArgs &a, const KVPrep &p, const CacheArgs &c, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_cache_append(const uint16_t *k, const uint16_t *v, const int32_t *positions, const int32_t *slots,
                               int n, int hkv, int pool_rows, double rope_base, uint16_t *k_pool, uint16_t *v_pool,
                               hipStream_t stream);
hipError_t launch_rope_table(float2 *table, int npos, double base, hipStream_t stream);
hipError_t launch_zero_f32(float *p, int n, hipStream_t stream);   // a fill kernel (no memset nodes)

// Head-group sizes (n_q_heads / n_kv_heads) with compiled kernels.
bool fwd_group_supported(int group);
bool bwd_group_supported(int group);
bool decode_group_supported(int group);

size_t fwd_workspace_bytes(int T, int hq, int hkv, int window);
size_t bwd_workspace_bytes(int T, int hq, int hkv, int window);
size_t bwd_workspace_bytes_ds(int T, int hq, int hkv, int window, int batch, int max_seqlen);   // 0: not available
size_t decode_workspace_bytes(int batch, int max_cache_len, int hq, int window, int nq = 1);
void decode_split_plan(int batch, int max_cache_len, int hq, int hkv, int window, int *splits, int *split_len);
// The same plan with at most as many splits as let the partials fit in cap bytes (laid out as
// decode_workspace_bytes lays them out); false when even one split does not fit.
bool decode_split_plan_capped(int batch, int max_cache_len, int hq, int window, int nq, size_t cap, int *splits,
                              int *split_len);

}  // namespace mimo
