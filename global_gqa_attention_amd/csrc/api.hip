// api.hip -- the extern "C" entry points declared in include/mimo_attn.h.
//
// Host-only argument checks (no device data is read), the per-device RoPE cos/sin table cache, workspace
// carving, and dispatch to the kernel launchers.  Nothing here allocates per call; the only allocation is
// a RoPE table the first time a (device, rope_base) pair needs more positions than cached.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "internal.hpp"
#include "mimo_attn.h"

namespace {

thread_local std::string g_last_error;

mimo_status_t fail(mimo_status_t s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

mimo_status_t ok()
{
    g_last_error.clear();
    return MIMO_OK;
}

mimo_status_t hip_fail(hipError_t e, const char *what)
{
    return fail(MIMO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- RoPE table cache: key (device, bits of rope_base) -> table of at least npos positions.
struct Table {
    float2 *ptr = nullptr;
    int npos = 0;
};
std::mutex g_mu;
std::map<std::pair<int, uint64_t>, Table> g_tables;
std::vector<std::pair<int, void *>> g_retired;  // grown-out tables, kept until release (may be in use)

mimo_status_t rope_table(double base, int need, hipStream_t stream, const float2 **out, int *npos)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    uint64_t bits;
    memcpy(&bits, &base, sizeof bits);
    std::lock_guard<std::mutex> lock(g_mu);
    Table &t = g_tables[{dev, bits}];
    if (t.npos < need) {
        int n = 4096;
        while (n < need) n = n < (1 << 30) ? n * 2 : need;
        float2 *p = nullptr;
        e = hipMalloc(&p, (size_t)n * 32 * sizeof(float2));
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(rope table)");
        e = mimo::launch_rope_table(p, n, base, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);  // other streams may use it right away
        if (e != hipSuccess) {
            (void)hipFree(p);
            return hip_fail(e, "building the rope table");
        }
        if (t.ptr) g_retired.push_back({dev, t.ptr});
        t.ptr = p;
        t.npos = n;
    }
    *out = t.ptr;
    *npos = t.npos;
    return MIMO_OK;
}

// ---- tracing: (name, start event, end event) per launched kernel
struct TraceRec {
    const char *name;
    hipEvent_t start, stop;
};
bool g_trace_on = false;
thread_local bool g_trace_off_here = false;   // set while an entry point that must not allocate runs
std::vector<TraceRec> g_trace;
std::vector<hipEvent_t> g_event_pool;
const char *g_trace_pending = nullptr;
hipEvent_t g_trace_start = nullptr;

hipEvent_t pool_event()
{
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

constexpr int kDQK = 192, kDV = 128;

mimo_status_t check_layer(const void *q, const void *k, const void *v, const int32_t *cu, int32_t batch,
                          int32_t T, int32_t max_seqlen, int32_t window, double rope_base, int32_t hq,
                          int32_t hkv)
{
    if (batch < 0) return fail(MIMO_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", batch);
    if (T < 0) return fail(MIMO_ERR_INVALID_ARG, "total_tokens must be >= 0 (got %d)", T);
    if (max_seqlen < 0) return fail(MIMO_ERR_INVALID_ARG, "max_seqlen must be >= 0 (got %d)", max_seqlen);
    if (T > 0 && max_seqlen == 0) return fail(MIMO_ERR_INVALID_ARG, "max_seqlen is 0 but total_tokens > 0");
    if (T > 0 && batch == 0) return fail(MIMO_ERR_INVALID_ARG, "total_tokens > 0 with batch 0");
    if (window < -1) return fail(MIMO_ERR_INVALID_ARG, "window must be -1 or >= 0 (got %d)", window);
    if (hq <= 0 || hkv <= 0) return fail(MIMO_ERR_INVALID_ARG, "head counts must be positive");
    if (hq % hkv != 0) return fail(MIMO_ERR_INVALID_ARG, "n_q_heads (%d) %% n_kv_heads (%d) != 0", hq, hkv);
    if (!(rope_base > 1.0) || !isfinite(rope_base))
        return fail(MIMO_ERR_INVALID_ARG, "rope_base must be finite and > 1 (got %g)", rope_base);
    if (T > 0 && (!q || !k || !v || !cu)) return fail(MIMO_ERR_INVALID_ARG, "null input pointer");
    if (batch > 0 && !cu) return fail(MIMO_ERR_INVALID_ARG, "cu_seqlens is null");
    if ((long long)T * hq * kDQK > (1LL << 40)) return fail(MIMO_ERR_UNSUPPORTED, "tensor too large");
    if (hq > 4096) return fail(MIMO_ERR_UNSUPPORTED, "n_q_heads above 4096 (got %d)", hq);
    return MIMO_OK;
}

}  // namespace

namespace mimo {
void trace_begin(const char *name, hipStream_t stream)
{
    if (!g_trace_on || g_trace_off_here) return;
    g_trace_start = pool_event();
    g_trace_pending = name;
    if (g_trace_start) (void)hipEventRecord(g_trace_start, stream);
}

void trace_end(hipStream_t stream)
{
    if (!g_trace_on || g_trace_off_here || !g_trace_start) return;
    hipEvent_t stop = pool_event();
    if (!stop) return;
    (void)hipEventRecord(stop, stream);
    g_trace.push_back({g_trace_pending, g_trace_start, stop});
    g_trace_start = nullptr;
}
}  // namespace mimo

extern "C" {

mimo_status_t mimo_attn_trace_enable(int enable)
{
    g_trace_on = enable != 0;
    return ok();
}

int32_t mimo_attn_trace_count(void) { return (int32_t)g_trace.size(); }

mimo_status_t mimo_attn_trace_read(int32_t i, const char **name, float *ms)
{
    if (i < 0 || i >= (int32_t)g_trace.size() || !name || !ms)
        return fail(MIMO_ERR_INVALID_ARG, "trace record %d out of range", i);
    TraceRec &r = g_trace[i];
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "reading a trace event");
    *name = r.name;
    return ok();
}

void mimo_attn_trace_clear(void)
{
    for (auto &r : g_trace) {
        (void)hipEventSynchronize(r.stop);
        g_event_pool.push_back(r.start);
        g_event_pool.push_back(r.stop);
    }
    g_trace.clear();
}

const char *mimo_attn_status_string(mimo_status_t s)
{
    switch (s) {
    case MIMO_OK: return "MIMO_OK";
    case MIMO_ERR_INVALID_ARG: return "MIMO_ERR_INVALID_ARG";
    case MIMO_ERR_UNSUPPORTED: return "MIMO_ERR_UNSUPPORTED";
    case MIMO_ERR_HIP: return "MIMO_ERR_HIP";
    case MIMO_ERR_WORKSPACE: return "MIMO_ERR_WORKSPACE";
    }
    return "MIMO_ERR_UNKNOWN";
}

const char *mimo_attn_last_error(void) { return g_last_error.c_str(); }

void mimo_attn_release(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto &kv : g_tables) {
        if (kv.second.ptr) {
            (void)hipSetDevice(kv.first.first);
            (void)hipFree(kv.second.ptr);
        }
    }
    for (auto &r : g_retired) {
        (void)hipSetDevice(r.first);
        (void)hipFree(r.second);
    }
    (void)hipSetDevice(cur);
    g_tables.clear();
    g_retired.clear();
}

mimo_status_t mimo_attn_fwd(const void *q, const void *k, const void *v, const float *sink,
                            const int32_t *cu_seqlens, int32_t batch, int32_t total_tokens,
                            int32_t max_seqlen, int32_t window, double rope_base, int32_t n_q_heads,
                            int32_t n_kv_heads, void *out, float *lse, void *q_rot, void *k_rot,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    mimo_status_t s = check_layer(q, k, v, cu_seqlens, batch, total_tokens, max_seqlen, window, rope_base,
                                  n_q_heads, n_kv_heads);
    if (s != MIMO_OK) return s;
    if (total_tokens > 0 && !out) return fail(MIMO_ERR_INVALID_ARG, "out is null");
    if (!mimo::fwd_group_supported(n_q_heads / n_kv_heads))
        return fail(MIMO_ERR_UNSUPPORTED, "no forward kernel for group size %d", n_q_heads / n_kv_heads);
    if (!mimo::fwd_stream_fits(total_tokens))
        return fail(MIMO_ERR_UNSUPPORTED, "total_tokens %d: the key stream passes the 32-bit copy offsets", total_tokens);
    if (total_tokens == 0) return ok();
    const size_t need = mimo::fwd_workspace_bytes(total_tokens, n_q_heads, n_kv_heads, window);
    if (!workspace || workspace_bytes < need)
        return fail(MIMO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    hipStream_t st = (hipStream_t)stream;
    mimo::FwdArgs a{};
    mimo::prep_carve(workspace, total_tokens, n_kv_heads, &a.P);
    a.P.k_rot = (uint16_t *)k_rot;
    s = rope_table(rope_base, max_seqlen, st, &a.L.rope, &a.L.rope_len);
    if (s != MIMO_OK) return s;
    a.L.q = (const uint16_t *)q;
    a.L.k = (const uint16_t *)k;
    a.L.v = (const uint16_t *)v;
    a.L.sink = sink;
    a.L.cu = cu_seqlens;
    a.L.batch = batch;
    a.L.T = total_tokens;
    a.L.window = window;
    a.L.hq = n_q_heads;
    a.L.hkv = n_kv_heads;
    a.L.scale_log2 = (float)(1.4426950408889634 / sqrt((double)kDQK));
    a.out = (uint16_t *)out;
    a.lse = lse;
    a.q_rot = (uint16_t *)q_rot;
    hipError_t e = mimo::launch_fwd(a, st);
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    return ok();
}

size_t mimo_attn_fwd_workspace_size(int32_t total_tokens, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t window)
{
    if (total_tokens < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || !mimo::fwd_stream_fits(total_tokens)) return 0;
    return mimo::fwd_workspace_bytes(total_tokens, n_q_heads, n_kv_heads, window);
}

size_t mimo_attn_prefill_cached_workspace_size(int32_t total_tokens, int32_t total_cache, int32_t n_kv_heads)
{
    if (total_tokens < 0 || total_cache < 0 || n_kv_heads <= 0) return 0;
    if (!mimo::fwd_stream_fits((long long)total_tokens + total_cache)) return 0;
    return mimo::prep_bytes(total_tokens + total_cache, n_kv_heads);
}

}  // extern "C"

namespace {
mimo_status_t prefill_over_cache(const void *q, const void *k, const void *v, const void *k_cache, const void *v_cache,
                                 const int32_t *page_table, const float *sink, const int32_t *cu_seqlens,
                                 const int32_t *cu_cache, const int32_t *positions, int32_t batch,
                                 int32_t total_tokens, int32_t total_cache, int32_t max_seqlen, int32_t max_position,
                                 int32_t window, double rope_base, int32_t n_q_heads, int32_t n_kv_heads, void *out,
                                 float *lse, void *workspace, size_t workspace_bytes, void *stream)
{
    mimo_status_t s = check_layer(q, k, v, cu_seqlens, batch, total_tokens, max_seqlen, window, rope_base,
                                  n_q_heads, n_kv_heads);
    if (s != MIMO_OK) return s;
    if (total_cache < 0) return fail(MIMO_ERR_INVALID_ARG, "total_cache must be >= 0 (got %d)", total_cache);
    if (!mimo::fwd_stream_fits((long long)total_tokens + total_cache))
        return fail(MIMO_ERR_UNSUPPORTED, "total_tokens + total_cache = %lld: the key stream passes the 32-bit copy "
                    "offsets", (long long)total_tokens + total_cache);
    if (max_position < max_seqlen)
        return fail(MIMO_ERR_INVALID_ARG, "max_position (%d) must be >= max_seqlen (%d)", max_position, max_seqlen);
    if (batch > 0 && (!cu_cache || !positions)) return fail(MIMO_ERR_INVALID_ARG, "cu_cache or positions is null");
    if (total_cache > 0 && (!k_cache || !v_cache)) return fail(MIMO_ERR_INVALID_ARG, "null cache pointer");
    if (total_tokens > 0 && !out) return fail(MIMO_ERR_INVALID_ARG, "out is null");
    if (!mimo::fwd_group_supported(n_q_heads / n_kv_heads))
        return fail(MIMO_ERR_UNSUPPORTED, "no forward kernel for group size %d", n_q_heads / n_kv_heads);
    if (total_tokens == 0) return ok();
    if ((long long)(total_tokens + total_cache) * n_kv_heads * kDQK > (1LL << 40))
        return fail(MIMO_ERR_UNSUPPORTED, "tensor too large");
    const size_t need = mimo::prep_bytes(total_tokens + total_cache, n_kv_heads);
    if (!workspace || workspace_bytes < need)
        return fail(MIMO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    hipStream_t st = (hipStream_t)stream;
    mimo::FwdArgs a{};
    mimo::prep_carve(workspace, total_tokens + total_cache, n_kv_heads, &a.P);
    s = rope_table(rope_base, max_position, st, &a.L.rope, &a.L.rope_len);
    if (s != MIMO_OK) return s;
    a.L.q = (const uint16_t *)q;
    a.L.k = (const uint16_t *)k;
    a.L.v = (const uint16_t *)v;
    a.L.sink = sink;
    a.L.cu = cu_seqlens;
    a.L.batch = batch;
    a.L.T = total_tokens;
    a.L.window = window;
    a.L.hq = n_q_heads;
    a.L.hkv = n_kv_heads;
    a.L.scale_log2 = (float)(1.4426950408889634 / sqrt((double)kDQK));
    a.C.k_cache = (const uint16_t *)k_cache;
    a.C.v_cache = (const uint16_t *)v_cache;
    a.C.cu_cache = cu_cache;
    a.C.page_table = page_table;
    a.C.positions = positions;
    a.C.Tc = total_cache;
    a.out = (uint16_t *)out;
    a.lse = lse;
    hipError_t e = mimo::launch_fwd(a, st);
    if (e != hipSuccess) return hip_fail(e, "cached prefill launch");
    return ok();
}
}  // namespace

extern "C" {

mimo_status_t mimo_attn_prefill_cached(const void *q, const void *k, const void *v, const void *k_cache,
                                       const void *v_cache, const float *sink, const int32_t *cu_seqlens,
                                       const int32_t *cu_cache, const int32_t *positions, int32_t batch,
                                       int32_t total_tokens, int32_t total_cache, int32_t max_seqlen,
                                       int32_t max_position, int32_t window, double rope_base,
                                       int32_t n_q_heads, int32_t n_kv_heads, void *out, float *lse,
                                       void *workspace, size_t workspace_bytes, void *stream)
{
    return prefill_over_cache(q, k, v, k_cache, v_cache, nullptr, sink, cu_seqlens, cu_cache, positions, batch,
                              total_tokens, total_cache, max_seqlen, max_position, window, rope_base, n_q_heads,
                              n_kv_heads, out, lse, workspace, workspace_bytes, stream);
}

mimo_status_t mimo_attn_prefill_paged(const void *q, const void *k, const void *v, const void *k_pool,
                                      const void *v_pool, const int32_t *page_table, const float *sink,
                                      const int32_t *cu_seqlens, const int32_t *cu_pages, const int32_t *positions,
                                      int32_t batch, int32_t total_tokens, int32_t total_pages, int32_t max_seqlen,
                                      int32_t max_position, int32_t window, double rope_base, int32_t n_q_heads,
                                      int32_t n_kv_heads, void *out, float *lse, void *workspace,
                                      size_t workspace_bytes, void *stream)
{
    if (total_pages > 0 && !page_table) return fail(MIMO_ERR_INVALID_ARG, "page_table is null");
    return prefill_over_cache(q, k, v, k_pool, v_pool, total_pages > 0 ? page_table : nullptr, sink, cu_seqlens,
                              cu_pages, positions, batch, total_tokens, total_pages, max_seqlen, max_position, window,
                              rope_base, n_q_heads, n_kv_heads, out, lse, workspace, workspace_bytes, stream);
}

mimo_status_t mimo_attn_cache_append(const void *k, const void *v, const int32_t *positions, const int32_t *slots,
                                     int32_t n_tokens, int32_t n_kv_heads, int32_t pool_rows, double rope_base,
                                     void *k_pool, void *v_pool, void *stream)
{
    if (n_tokens < 0) return fail(MIMO_ERR_INVALID_ARG, "n_tokens must be >= 0 (got %d)", n_tokens);
    if (n_kv_heads <= 0) return fail(MIMO_ERR_INVALID_ARG, "n_kv_heads must be positive");
    if (pool_rows < 0) return fail(MIMO_ERR_INVALID_ARG, "pool_rows must be >= 0");
    if (!(rope_base > 1.0) || !isfinite(rope_base))
        return fail(MIMO_ERR_INVALID_ARG, "rope_base must be finite and > 1 (got %g)", rope_base);
    if (n_tokens == 0) return ok();
    if (!k || !v || !positions || !slots || !k_pool || !v_pool)
        return fail(MIMO_ERR_INVALID_ARG, "null pointer among k/v/positions/slots/k_pool/v_pool");
    if (n_kv_heads > 65535) return fail(MIMO_ERR_UNSUPPORTED, "too many KV heads");
    hipError_t e = mimo::launch_cache_append((const uint16_t *)k, (const uint16_t *)v, positions, slots, n_tokens,
                                             n_kv_heads, pool_rows, rope_base, (uint16_t *)k_pool,
                                             (uint16_t *)v_pool, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "cache append launch");
    return ok();
}

size_t mimo_attn_bwd_workspace_size(int32_t total_tokens, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t window)
{
    if (total_tokens < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || !mimo::bwd_stream_fits(total_tokens)) return 0;
    return mimo::bwd_workspace_bytes(total_tokens, n_q_heads, n_kv_heads, window);
}

size_t mimo_attn_bwd_workspace_size_fast(int32_t total_tokens, int32_t batch, int32_t max_seqlen,
                                         int32_t n_q_heads, int32_t n_kv_heads, int32_t window)
{
    if (total_tokens < 0 || batch < 0 || max_seqlen < 0 || n_q_heads <= 0 || n_kv_heads <= 0) return 0;
    if (!mimo::bwd_stream_fits(total_tokens)) return 0;
    const size_t ds = mimo::bwd_workspace_bytes_ds(total_tokens, n_q_heads, n_kv_heads, window, batch, max_seqlen);
    return ds ? ds : mimo::bwd_workspace_bytes(total_tokens, n_q_heads, n_kv_heads, window);
}

mimo_status_t mimo_attn_bwd(const void *q, const void *k, const void *v, const float *sink,
                            const void *out, const float *lse, const void *dout, const void *q_rot,
                            const void *k_rot, const int32_t *cu_seqlens, int32_t batch, int32_t total_tokens,
                            int32_t max_seqlen, int32_t window, double rope_base, int32_t n_q_heads,
                            int32_t n_kv_heads, void *dq, void *dk, void *dv, float *dsink,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    mimo_status_t s = check_layer(q, k, v, cu_seqlens, batch, total_tokens, max_seqlen, window, rope_base,
                                  n_q_heads, n_kv_heads);
    if (s != MIMO_OK) return s;
    if ((sink == nullptr) != (dsink == nullptr))
        return fail(MIMO_ERR_INVALID_ARG, "dsink must be given exactly when sink is given");
    if (total_tokens > 0 && (!out || !lse || !dout || !dq || !dk || !dv))
        return fail(MIMO_ERR_INVALID_ARG, "null pointer among out/lse/dout/dq/dk/dv");
    if (!mimo::bwd_group_supported(n_q_heads / n_kv_heads))
        return fail(MIMO_ERR_UNSUPPORTED, "no backward kernel for group size %d", n_q_heads / n_kv_heads);
    if (!mimo::bwd_stream_fits(total_tokens))
        return fail(MIMO_ERR_UNSUPPORTED, "total_tokens %d: the key stream passes the 32-bit copy offsets", total_tokens);
    const size_t need = mimo::bwd_workspace_bytes(total_tokens, n_q_heads, n_kv_heads, window);
    if (total_tokens > 0 && (!workspace || workspace_bytes < need))
        return fail(MIMO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    hipStream_t st = (hipStream_t)stream;
    if (total_tokens == 0) {
        if (dsink) {
            hipError_t e = mimo::launch_zero_f32(dsink, n_q_heads, st);
            if (e != hipSuccess) return hip_fail(e, "clearing dsink");
        }
        return ok();
    }
    mimo::BwdArgs a{};
    s = rope_table(rope_base, max_seqlen, st, &a.L.rope, &a.L.rope_len);
    if (s != MIMO_OK) return s;
    a.L.q = (const uint16_t *)q;
    a.L.k = (const uint16_t *)k;
    a.L.v = (const uint16_t *)v;
    a.L.sink = sink;
    a.L.cu = cu_seqlens;
    a.L.batch = batch;
    a.L.T = total_tokens;
    a.L.window = window;
    a.L.hq = n_q_heads;
    a.L.hkv = n_kv_heads;
    a.L.scale_log2 = (float)(1.4426950408889634 / sqrt((double)kDQK));
    a.out = (const uint16_t *)out;
    a.dout = (const uint16_t *)dout;
    a.lse = lse;
    a.dq = (uint16_t *)dq;
    a.dk = (uint16_t *)dk;
    a.dv = (uint16_t *)dv;
    a.dsink = dsink;
    const size_t ds_need = mimo::bwd_workspace_bytes_ds(total_tokens, n_q_heads, n_kv_heads, window, batch,
                                                        max_seqlen);
    const bool stored_ds = ds_need > 0 && workspace_bytes >= ds_need;
    mimo::bwd_carve(workspace, total_tokens, n_q_heads, n_kv_heads, &a, stored_ds, batch, max_seqlen);
    a.qr_rows = a.T_pad;
    a.qr_given = q_rot != nullptr;
    if (q_rot) {   // the forward's rotated q replaces the workspace copy (read only)
        a.W.qr = (uint16_t *)q_rot;
        a.qr_rows = total_tokens;
    }
    a.kr_rows = a.T_pad;
    a.kr_given = k_rot != nullptr && stored_ds;
    if (a.kr_given) {   // the forward's rotated k replaces the workspace's row copy (read only)
        a.W.kr = (uint16_t *)k_rot;
        a.kr_rows = total_tokens;
    }
    if (stored_ds) a.ds_cap = (int64_t)((ds_need - (size_t)((char *)a.ds - (char *)workspace)) / 2048);
    hipError_t e = mimo::launch_bwd(a, st);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return ok();
}

size_t mimo_attn_decode_workspace_size(int32_t batch, int32_t max_cache_len, int32_t n_q_heads,
                                       int32_t window)
{
    if (batch < 0 || max_cache_len < 0 || n_q_heads <= 0) return 0;
    return mimo::decode_workspace_bytes(batch, max_cache_len, n_q_heads, window);
}

}  // extern "C"

// ---- scratch for callers that cannot allocate (mimo_attn_decode_paged_noalloc): the split-KV partials live
// in this array, one copy per device for the life of the process.  Host code never passes the array's own
// name to a kernel (on the host it stands for nothing on the device); each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_addr;

mimo_status_t scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch_addr.find(dev);
    if (it == g_scratch_addr.end()) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MIMO_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
        it = g_scratch_addr.emplace(dev, p).first;
    }
    *out = it->second;
    return MIMO_OK;
}

// Decode (nq = 1, k_new/v_new given) or verify (nq draft tokens whose keys are the last nq cache rows,
// k_new == v_new == nullptr) over a contiguous or paged cache.
mimo_status_t decode_over_cache(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                                const void *v_cache, const int32_t *page_table, const int32_t *cu_cache,
                                const int32_t *positions, const float *sink, int32_t batch, int32_t nq,
                                int32_t max_cache_len, int32_t window, double rope_base, int32_t n_q_heads,
                                int32_t n_kv_heads, void *out, void *workspace, size_t workspace_bytes, void *stream,
                                bool use_scratch = false)
{
    const bool verify = k_new == nullptr;
    if (nq < 1 || (!verify && nq != 1)) return fail(MIMO_ERR_INVALID_ARG, "query tokens per sequence must be >= 1");
    if (verify && batch > 0 && max_cache_len < nq)
        return fail(MIMO_ERR_INVALID_ARG, "max_cache_len (%d) must cover the %d draft rows", max_cache_len, nq);
    if (batch < 0) return fail(MIMO_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", batch);
    if (max_cache_len < 0) return fail(MIMO_ERR_INVALID_ARG, "max_cache_len must be >= 0");
    if (window < -1) return fail(MIMO_ERR_INVALID_ARG, "window must be -1 or >= 0 (got %d)", window);
    if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0)
        return fail(MIMO_ERR_INVALID_ARG, "bad head counts %d / %d", n_q_heads, n_kv_heads);
    if (!(rope_base > 1.0) || !isfinite(rope_base))
        return fail(MIMO_ERR_INVALID_ARG, "rope_base must be finite and > 1 (got %g)", rope_base);
    if (batch == 0) return ok();
    if (!q || (!verify && !v_new) || !cu_cache || !positions || !out)
        return fail(MIMO_ERR_INVALID_ARG, "null pointer among q/k_new/v_new/cu_cache/positions/out");
    if ((long long)batch * nq * n_q_heads > 0x7fffffffLL) return fail(MIMO_ERR_UNSUPPORTED, "too many query rows");
    if (max_cache_len > 0 && (!k_cache || !v_cache)) return fail(MIMO_ERR_INVALID_ARG, "null cache pointer");
    if (!mimo::decode_group_supported(n_q_heads / n_kv_heads))
        return fail(MIMO_ERR_UNSUPPORTED, "no decode kernel for group size %d", n_q_heads / n_kv_heads);
    const int wplan = verify && window >= 0 ? window + nq : window;   // rows a query can see
    int splits = 0, split_len = 0;
    if (use_scratch) {
        // the scratch array instead of a workspace: fewer, longer splits when the usual plan's partials do
        // not fit in it
        if (!mimo::decode_split_plan_capped(batch, max_cache_len, n_q_heads, wplan, nq, kScratchBytes, &splits,
                                            &split_len))
            return fail(MIMO_ERR_UNSUPPORTED, "batch %d x %d query heads: the split partials need more than the "
                        "%zu-byte scratch array", batch, n_q_heads, kScratchBytes);
        mimo_status_t st = scratch_address(&workspace);
        if (st != MIMO_OK) return st;
        workspace_bytes = kScratchBytes;
    } else {
        const size_t need = mimo::decode_workspace_bytes(batch, max_cache_len, n_q_heads, wplan, nq);
        if (need > 0 && (!workspace || workspace_bytes < need))
            return fail(MIMO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
        mimo::decode_split_plan(batch, max_cache_len, n_q_heads, n_kv_heads, wplan, &splits, &split_len);
    }
    mimo::DecodeArgs a{};
    a.q = (const uint16_t *)q;
    a.k_new = (const uint16_t *)k_new;
    a.v_new = (const uint16_t *)v_new;
    a.k_cache = (const uint16_t *)k_cache;
    a.v_cache = (const uint16_t *)v_cache;
    a.cu_cache = cu_cache;
    a.page_table = page_table;
    a.positions = positions;
    a.sink = sink;
    a.out = (uint16_t *)out;
    a.batch = batch;
    a.nq = nq;
    a.window = window;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    a.rope_base = rope_base;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)kDQK));
    a.splits = splits;
    a.split_len = split_len;
    char *ws = (char *)workspace;
    a.part_o = (float *)ws;
    size_t off = ((size_t)batch * nq * n_q_heads * a.splits * kDV * sizeof(float) + 255) & ~(size_t)255;
    a.part_ml = (float *)(ws + off);
    hipError_t e = mimo::launch_decode(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
}
}  // namespace

extern "C" {

mimo_status_t mimo_attn_decode(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                               const void *v_cache, const int32_t *cu_cache, const int32_t *positions,
                               const float *sink, int32_t batch, int32_t max_cache_len, int32_t window,
                               double rope_base, int32_t n_q_heads, int32_t n_kv_heads, void *out,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    if (batch > 0 && !k_new) return fail(MIMO_ERR_INVALID_ARG, "k_new is null");
    return decode_over_cache(q, k_new, v_new, k_cache, v_cache, nullptr, cu_cache, positions, sink, batch, 1,
                             max_cache_len, window, rope_base, n_q_heads, n_kv_heads, out, workspace,
                             workspace_bytes, stream);
}

mimo_status_t mimo_attn_decode_paged(const void *q, const void *k_new, const void *v_new, const void *k_pool,
                                     const void *v_pool, const int32_t *page_table, const int32_t *cu_pages,
                                     const int32_t *positions, const float *sink, int32_t batch,
                                     int32_t max_cache_len, int32_t window, double rope_base, int32_t n_q_heads,
                                     int32_t n_kv_heads, void *out, void *workspace, size_t workspace_bytes,
                                     void *stream)
{
    if (batch > 0 && max_cache_len > 0 && !page_table) return fail(MIMO_ERR_INVALID_ARG, "page_table is null");
    if (batch > 0 && !k_new) return fail(MIMO_ERR_INVALID_ARG, "k_new is null");
    return decode_over_cache(q, k_new, v_new, k_pool, v_pool, max_cache_len > 0 ? page_table : nullptr, cu_pages,
                             positions, sink, batch, 1, max_cache_len, window, rope_base, n_q_heads, n_kv_heads, out,
                             workspace, workspace_bytes, stream);
}

mimo_status_t mimo_attn_decode_paged_noalloc(const void *q, const void *k_new, const void *v_new, const void *k_pool,
                                             const void *v_pool, const int32_t *page_table, const int32_t *cu_pages,
                                             const int32_t *positions, const float *sink, int32_t batch,
                                             int32_t max_cache_len, int32_t window, double rope_base,
                                             int32_t n_q_heads, int32_t n_kv_heads, void *out, void *stream)
{
    if (batch > 0 && max_cache_len > 0 && !page_table) return fail(MIMO_ERR_INVALID_ARG, "page_table is null");
    if (batch > 0 && !k_new) return fail(MIMO_ERR_INVALID_ARG, "k_new is null");
    g_trace_off_here = true;   // tracing would create HIP events
    const mimo_status_t s = decode_over_cache(q, k_new, v_new, k_pool, v_pool, max_cache_len > 0 ? page_table : nullptr,
                                              cu_pages, positions, sink, batch, 1, max_cache_len, window, rope_base,
                                              n_q_heads, n_kv_heads, out, nullptr, 0, stream, true);
    g_trace_off_here = false;
    return s;
}

size_t mimo_attn_verify_workspace_size(int32_t batch, int32_t n_query, int32_t max_cache_len, int32_t n_q_heads,
                                       int32_t window)
{
    if (batch < 0 || n_query < 1 || max_cache_len < 0 || n_q_heads <= 0 || window < -1) return 0;
    return mimo::decode_workspace_bytes(batch, max_cache_len, n_q_heads, window >= 0 ? window + n_query : window,
                                        n_query);
}

mimo_status_t mimo_attn_verify_paged(const void *q, const void *k_pool, const void *v_pool, const int32_t *page_table,
                                     const int32_t *cu_pages, const int32_t *positions, const float *sink,
                                     int32_t batch, int32_t n_query, int32_t max_cache_len, int32_t window,
                                     double rope_base, int32_t n_q_heads, int32_t n_kv_heads, void *out,
                                     void *workspace, size_t workspace_bytes, void *stream)
{
    if (batch > 0 && !page_table) return fail(MIMO_ERR_INVALID_ARG, "page_table is null");
    if (batch > 0 && (!k_pool || !v_pool)) return fail(MIMO_ERR_INVALID_ARG, "null pool pointer");
    return decode_over_cache(q, nullptr, nullptr, k_pool, v_pool, page_table, cu_pages, positions, sink, batch,
                             n_query, max_cache_len, window, rope_base, n_q_heads, n_kv_heads, out, workspace,
                             workspace_bytes, stream);
}

}  // extern "C"
