// C ABI of libmedusa: argument validation, workspace layout and kernel orchestration for
// one Medusa decode step.  Every check that the host can make happens before anything is
// enqueued; nothing here allocates device memory or synchronises a stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "advance.hpp"
#include "plan_impl.hpp"
#include "probe.hpp"
#include "rope.hpp"

using namespace medusa;

namespace {

thread_local int g_last_hip_error = 0;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
size_t esize(medusa_dtype dt) { return dt == MEDUSA_BF16 ? 2 : 4; }
bool dtype_ok(medusa_dtype dt) { return dt == MEDUSA_BF16 || dt == MEDUSA_F32; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int n_tiles_for(medusa_dtype dt, int M, int epi, int N, int K) {
    const int rows = gemm_rows_per_tile(dt, M, epi, K, N);
    return (N + rows - 1) / rows;
}

// Workspace carving: a running offset over the caller's buffer.
struct Carver {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    }
};

struct HeadsLayout {
    size_t u = 0, part_val[kMaxProblems] = {}, part_idx[kMaxProblems] = {};
    size_t total = 0;
    int n_tiles = 0;
};

HeadsLayout heads_layout(medusa_dtype dt, int B, int H, int V, int K, int s_max, bool with_u) {
    HeadsLayout L;
    Carver c;
    if (with_u) L.u = c.take((size_t)B * K * H * esize(dt));
    L.n_tiles = n_tiles_for(dt, B, EPI_TOPS, V, H);
    for (int p = 0; p <= K; ++p) {
        const size_t n = (size_t)B * L.n_tiles * (p < K ? s_max : 1);
        L.part_val[p] = c.take(n * sizeof(float));
        L.part_idx[p] = c.take(n * sizeof(int32_t));
    }
    L.total = c.off;
    return L;
}

struct VerifyLayout {
    size_t part_val = 0, part_idx = 0, node_arg = 0;
    size_t part_z = 0, part_s = 0, cand_logit = 0, node_max = 0, node_z = 0, node_tau = 0;
    size_t total = 0;
    int n_tiles = 0;
};

// Greedy verification needs the per-tile argmax partials; typical acceptance adds the
// per-tile softmax sums and one candidate logit per node (same tiles: EPI_TYPICAL shares
// EPI_ARGMAX's kernels and tile sizes).
VerifyLayout verify_layout(medusa_dtype dt, int M, int V, int H, bool typical = false) {
    VerifyLayout L;
    Carver c;
    L.n_tiles = n_tiles_for(dt, M, EPI_ARGMAX, V, H);
    L.part_val = c.take((size_t)M * L.n_tiles * sizeof(float));
    L.part_idx = c.take((size_t)M * L.n_tiles * sizeof(int32_t));
    L.node_arg = c.take((size_t)M * sizeof(int32_t));        // when the caller wants none
    if (typical) {
        L.part_z = c.take((size_t)M * L.n_tiles * sizeof(float));
        L.part_s = c.take((size_t)M * L.n_tiles * sizeof(float));
        L.cand_logit = c.take((size_t)M * sizeof(float));
        L.node_max = c.take((size_t)M * sizeof(float));
        L.node_z = c.take((size_t)M * sizeof(float));
        L.node_tau = c.take((size_t)M * sizeof(float));
    }
    L.total = c.off;
    return L;
}

hipError_t timed_gemm(const char* name, medusa_dtype dt, int epi, GemmBatch& b, hipStream_t s) {
    prof_begin(name, s);
    hipError_t e = gemm_launch(dt, epi, b, s);
    prof_end(s);
    return e;
}

}  // namespace

medusa_status medusa_internal_device_check() {
    static std::once_flag once;
    static int count = 0;
    std::call_once(once, [] {
        int n = 0;
        if (hipGetDeviceCount(&n) != hipSuccess) n = 0;
        count = n;
    });
    return count > 0 ? MEDUSA_OK : MEDUSA_ERR_NO_DEVICE;
}

medusa_status medusa_internal_hip_error(hipError_t e) {
    g_last_hip_error = (int)e;
    return MEDUSA_ERR_HIP;
}

extern "C" {

const char* medusa_status_string(medusa_status st) {
    switch (st) {
        case MEDUSA_OK: return "ok";
        case MEDUSA_ERR_NULL: return "null pointer";
        case MEDUSA_ERR_SHAPE: return "bad shape";
        case MEDUSA_ERR_UNSUPPORTED: return "unsupported dtype or size";
        case MEDUSA_ERR_TREE: return "malformed tree";
        case MEDUSA_ERR_WORKSPACE: return "workspace too small";
        case MEDUSA_ERR_NO_DEVICE: return "no HIP device";
        case MEDUSA_ERR_HIP: return "HIP runtime error";
        case MEDUSA_ERR_PLAN_NOT_ON_DEVICE: return "plan not uploaded";
    }
    return "unknown status";
}

int medusa_last_hip_error(void) { return g_last_hip_error; }
int medusa_version(void) { return 1; }

// ------------------------------------------------------------------ 1. heads

size_t medusa_heads_workspace(medusa_dtype dt, int B, int H, int V, int K, int s_max) {
    if (!dtype_ok(dt) || B < 1 || H < 1 || V < 1 || K < 1 || K > MEDUSA_MAX_HEADS || s_max < 1)
        return 0;
    return heads_layout(dt, B, H, V, K, s_max, true).total;
}

medusa_status medusa_heads_forward(medusa_dtype dt, int B, int H, int V, int K,
                                   const void* hidden, const void* w1, const void* b1,
                                   const void* w2, const void* w_lm, const int32_t* s,
                                   int s_max, int32_t* topk_ids, float* topk_vals,
                                   int32_t* root_ids, void* u_out, float* logits, void* ws,
                                   size_t ws_bytes, void* stream) {
    if (!hidden || !w1 || !b1 || !w2 || !s || !topk_ids || !topk_vals) return MEDUSA_ERR_NULL;
    if (w_lm && !root_ids) return MEDUSA_ERR_NULL;
    if (!dtype_ok(dt)) return MEDUSA_ERR_UNSUPPORTED;
    if (B < 1 || B > 64 || K < 1 || K > MEDUSA_MAX_HEADS || H < 32 || H > 16384 || H % 32 != 0 ||
        V < 1)
        return MEDUSA_ERR_SHAPE;
    int smax_seen = 0;
    for (int k = 0; k < K; ++k) {
        if (s[k] < 1 || s[k] > MEDUSA_MAX_TOPK || s[k] > V) return MEDUSA_ERR_UNSUPPORTED;
        smax_seen = s[k] > smax_seen ? s[k] : smax_seen;
    }
    if (s_max < smax_seen || s_max > MEDUSA_MAX_TOPK) return MEDUSA_ERR_SHAPE;
    if (!aligned16(hidden) || !aligned16(w1) || !aligned16(w2) || (w_lm && !aligned16(w_lm)) ||
        (u_out && !aligned16(u_out)))
        return MEDUSA_ERR_SHAPE;
    const HeadsLayout L = heads_layout(dt, B, H, V, K, s_max, u_out == nullptr);
    if (L.n_tiles > 2048) return MEDUSA_ERR_SHAPE;
    if (!ws || ws_bytes < L.total) return MEDUSA_ERR_WORKSPACE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;

    hipStream_t strm = static_cast<hipStream_t>(stream);
    unsigned char* wsb = static_cast<unsigned char*>(ws);
    const size_t es = esize(dt);
    unsigned char* u = u_out ? static_cast<unsigned char*>(u_out) : wsb + L.u;

    // A1: u_bk = rnd(h_b + SiLU(W1_k h_b + b1_k)) for all heads in one launch
    GemmBatch ffn{};
    ffn.n_problems = K;
    ffn.M = B;
    ffn.K = H;
    const int ffn_tiles = n_tiles_for(dt, B, EPI_STORE, H, H);
    for (int k = 0; k < K; ++k) {
        GemmProblem& p = ffn.p[k];
        p.W = static_cast<const unsigned char*>(w1) + (size_t)k * H * H * es;
        p.X = hidden;
        p.x_stride = H;
        p.N = H;
        p.tile_begin = k * ffn_tiles;
        p.n_tiles = ffn_tiles;
        p.out = u + (size_t)k * H * es;
        p.ldo = (long long)K * H;
        p.bias = static_cast<const unsigned char*>(b1) + (size_t)k * H * es;
        p.silu = 1;
        p.res = hidden;
        p.res_stride = H;
    }
    ffn.total_tiles = K * ffn_tiles;
    hipError_t e = timed_gemm("heads_ffn", dt, EPI_STORE, ffn, strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);

    // A2 + A3: logits_bk = W2_k u_bk with a fused per-tile top-s; the bootstrap root uses
    // the same code path on (W_lm, h) with s = 1.
    GemmBatch voc{};
    const int P = K + (w_lm ? 1 : 0);
    voc.n_problems = P;
    voc.M = B;
    voc.K = H;
    for (int p = 0; p < P; ++p) {
        GemmProblem& g = voc.p[p];
        const bool root = p == K;
        g.W = root ? w_lm : static_cast<const void*>(static_cast<const unsigned char*>(w2) +
                                                     (size_t)p * V * H * es);
        g.X = root ? hidden : static_cast<const void*>(u + (size_t)p * H * es);
        g.x_stride = root ? H : (long long)K * H;
        g.N = V;
        g.tile_begin = p * L.n_tiles;
        g.n_tiles = L.n_tiles;
        g.s = root ? 1 : s[p];
        g.part_val = reinterpret_cast<float*>(wsb + L.part_val[p]);
        g.part_idx = reinterpret_cast<int32_t*>(wsb + L.part_idx[p]);
        g.logits = logits ? logits + (size_t)p * V : nullptr;
        g.logits_ld = (long long)(K + 1) * V;
    }
    voc.total_tiles = P * L.n_tiles;
    e = timed_gemm("heads_vocab", dt, EPI_TOPS, voc, strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);

    MergeBatch mg{};
    mg.n_problems = P;
    mg.M = B;
    for (int p = 0; p < P; ++p) {
        MergeProblem& m = mg.p[p];
        const bool root = p == K;
        m.part_val = voc.p[p].part_val;
        m.part_idx = voc.p[p].part_idx;
        m.n_tiles = L.n_tiles;
        m.s = voc.p[p].s;
        m.out_ids = root ? root_ids : topk_ids + (size_t)p * s_max;
        m.out_vals = root ? nullptr : topk_vals + (size_t)p * s_max;
        m.out_ld = root ? 1 : (long long)K * s_max;
        m.s_pad = root ? 1 : s_max;
    }
    prof_begin("heads_merge", strm);
    e = topk_merge_launch(mg, strm);
    prof_end(strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    return MEDUSA_OK;
}

// ------------------------------------------------------------------ 2. tree

medusa_status medusa_build_tree(const medusa_tree_plan* plan, int B, int K, int s_max,
                                const int32_t* s, const int32_t* root_ids,
                                const int32_t* topk_ids, const int32_t* prefix_lens,
                                int32_t* node_tokens, int32_t* position_ids, void* stream) {
    if (!plan || !s || !root_ids || !topk_ids || !node_tokens) return MEDUSA_ERR_NULL;
    if (B < 1 || K < 1 || K > MEDUSA_MAX_HEADS || s_max < 1 || s_max > MEDUSA_MAX_TOPK)
        return MEDUSA_ERR_SHAPE;
    if (plan->max_depth > K) return MEDUSA_ERR_TREE;
    for (int k = 0; k < K; ++k)
        if (s[k] < 1 || s[k] > s_max) return MEDUSA_ERR_SHAPE;
    for (int i = 1; i < plan->n_nodes; ++i)
        if (plan->rank[i] >= s[plan->depth[i] - 1]) return MEDUSA_ERR_TREE;
    if (!plan->dev) return MEDUSA_ERR_PLAN_NOT_ON_DEVICE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    hipStream_t strm = static_cast<hipStream_t>(stream);
    prof_begin("build_tree", strm);
    hipError_t e = build_tree_launch(medusa_internal_device_plan(plan), B, K, s_max, root_ids,
                                     topk_ids, prefix_lens, node_tokens, position_ids, strm);
    prof_end(strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    return MEDUSA_OK;
}

// ------------------------------------------------------------------ 3. tree attention

size_t medusa_attention_workspace(const medusa_tree_plan* plan, medusa_dtype dt, int B, int Hq,
                                  int Hkv, int d, int Lcap) {
    if (!plan || !dtype_ok(dt) || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Lcap < 0 ||
        (d != 64 && d != 128))
        return 0;
    return attn_workspace_bytes(attn_shape(dt, B, plan->n_nodes, Hq, Hkv, d, Lcap));
}

medusa_status medusa_tree_attention(const medusa_tree_plan* plan, medusa_dtype dt, int B, int Hq,
                                    int Hkv, int d, int Lcap, float scale, const void* q,
                                    const void* k_tree, const void* v_tree, const void* k_cache,
                                    const void* v_cache, const int32_t* prefix_lens, void* out,
                                    void* ws, size_t ws_bytes, void* stream) {
    if (!plan || !q || !k_tree || !v_tree || !prefix_lens || !out) return MEDUSA_ERR_NULL;
    if (Lcap > 0 && (!k_cache || !v_cache)) return MEDUSA_ERR_NULL;
    if (!dtype_ok(dt)) return MEDUSA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return MEDUSA_ERR_UNSUPPORTED;
    if (B < 1 || B > 4096 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Hq > 1024 || Lcap < 0 ||
        Lcap > (1 << 20))
        return MEDUSA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out) ||
        (Lcap > 0 && (!aligned16(k_cache) || !aligned16(v_cache))))
        return MEDUSA_ERR_SHAPE;
    const AttnShape sh = attn_shape(dt, B, plan->n_nodes, Hq, Hkv, d, Lcap);
    if (!ws || ws_bytes < attn_workspace_bytes(sh)) return MEDUSA_ERR_WORKSPACE;
    if (!plan->dev) return MEDUSA_ERR_PLAN_NOT_ON_DEVICE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    if (!(scale > 0.f)) scale = 1.0f / std::sqrt((float)d);
    hipError_t e = attention_launch(dt, sh, medusa_internal_device_plan(plan), scale, q, k_tree,
                                    v_tree, k_cache, v_cache, prefix_lens, out, ws,
                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    return MEDUSA_OK;
}

// ------------------------------------------------------------------ 4. verify + accept

size_t medusa_verify_workspace(const medusa_tree_plan* plan, medusa_dtype dt, int B, int H, int V) {
    if (!plan || !dtype_ok(dt) || B < 1 || H < 1 || V < 1) return 0;
    return verify_layout(dt, B * plan->n_nodes, V, H).total;
}

medusa_status medusa_verify_accept(const medusa_tree_plan* plan, medusa_dtype dt, int B, int H,
                                   int V, const void* node_hidden, const void* w_lm,
                                   const int32_t* node_tokens, int32_t* node_argmax,
                                   int32_t* accept_len, int32_t* accept_nodes,
                                   int32_t* accept_tokens, float* logits, void* ws,
                                   size_t ws_bytes, void* stream) {
    return medusa::verify_accept_impl(plan, dt, B, H, V, node_hidden, w_lm, node_tokens,
                                      node_argmax, accept_len, accept_nodes, accept_tokens,
                                      logits, ws, ws_bytes, stream);
}

}  // extern "C"

// Greedy verification and acceptance on a caller-given scratch area (the workspace, or the
// library's static scratch in medusa_verify_accept_noalloc).
medusa_status medusa::verify_accept_impl(const medusa_tree_plan* plan, medusa_dtype dt, int B,
                                         int H, int V, const void* node_hidden, const void* w_lm,
                                         const int32_t* node_tokens, int32_t* node_argmax,
                                         int32_t* accept_len, int32_t* accept_nodes,
                                         int32_t* accept_tokens, float* logits, void* ws,
                                         size_t ws_bytes, void* stream) {
    if (!plan || !node_hidden || !w_lm || !node_tokens || !accept_len || !accept_nodes ||
        !accept_tokens)
        return MEDUSA_ERR_NULL;
    if (!dtype_ok(dt)) return MEDUSA_ERR_UNSUPPORTED;
    if (B < 1 || B > 4096 || H < 32 || H > 16384 || H % 32 != 0 || V < 1) return MEDUSA_ERR_SHAPE;
    if (!aligned16(node_hidden) || !aligned16(w_lm)) return MEDUSA_ERR_SHAPE;
    const int M = B * plan->n_nodes;
    const VerifyLayout L = verify_layout(dt, M, V, H);
    if (!ws || ws_bytes < L.total) return MEDUSA_ERR_WORKSPACE;
    if (!plan->dev) return MEDUSA_ERR_PLAN_NOT_ON_DEVICE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    hipStream_t strm = static_cast<hipStream_t>(stream);
    unsigned char* wsb = static_cast<unsigned char*>(ws);
    float* pv = reinterpret_cast<float*>(wsb + L.part_val);
    int32_t* pi = reinterpret_cast<int32_t*>(wsb + L.part_idx);

    GemmBatch g{};
    g.n_problems = 1;
    g.M = M;
    g.K = H;
    GemmProblem& p = g.p[0];
    p.W = w_lm;
    p.X = node_hidden;
    p.x_stride = H;
    p.N = V;
    p.tile_begin = 0;
    p.n_tiles = L.n_tiles;
    p.s = 1;
    p.part_val = pv;
    p.part_idx = pi;
    p.logits = logits;
    p.logits_ld = V;
    g.total_tiles = L.n_tiles;
    hipError_t e = timed_gemm("verify_lmhead", dt, EPI_ARGMAX, g, strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    prof_begin("verify_accept", strm);
    int32_t* arg = node_argmax ? node_argmax : reinterpret_cast<int32_t*>(wsb + L.node_arg);
    e = accept_launch(medusa_internal_device_plan(plan), B, L.n_tiles, pv, pi, node_tokens,
                      arg, accept_len, accept_nodes, accept_tokens, strm);
    prof_end(strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    return MEDUSA_OK;
}

extern "C" {

size_t medusa_verify_typical_workspace(const medusa_tree_plan* plan, medusa_dtype dt, int B,
                                       int H, int V) {
    if (!plan || !dtype_ok(dt) || B < 1 || H < 1 || V < 1) return 0;
    return verify_layout(dt, B * plan->n_nodes, V, H, true).total;
}

medusa_status medusa_verify_accept_typical(const medusa_tree_plan* plan, medusa_dtype dt, int B,
                                           int H, int V, const void* node_hidden, const void* w_lm,
                                           const int32_t* node_tokens, float temperature,
                                           float epsilon, float delta, int32_t* node_argmax,
                                           float* node_prob, float* node_tau, int32_t* accept_len,
                                           int32_t* accept_nodes, int32_t* accept_tokens,
                                           float* logits, void* ws, size_t ws_bytes,
                                           void* stream) {
    if (!plan || !node_hidden || !w_lm || !node_tokens || !accept_len || !accept_nodes ||
        !accept_tokens)
        return MEDUSA_ERR_NULL;
    if (!dtype_ok(dt)) return MEDUSA_ERR_UNSUPPORTED;
    if (B < 1 || B > 4096 || H < 32 || H > 16384 || H % 32 != 0 || V < 1) return MEDUSA_ERR_SHAPE;
    if (!(temperature >= 1e-6f && temperature <= 1e6f) || !(epsilon >= 0.f) ||
        !(delta >= 0.f) || !std::isfinite(epsilon) || !std::isfinite(delta))
        return MEDUSA_ERR_SHAPE;
    if (!aligned16(node_hidden) || !aligned16(w_lm)) return MEDUSA_ERR_SHAPE;
    const int M = B * plan->n_nodes;
    const VerifyLayout L = verify_layout(dt, M, V, H, true);
    if (!ws || ws_bytes < L.total) return MEDUSA_ERR_WORKSPACE;
    if (!plan->dev) return MEDUSA_ERR_PLAN_NOT_ON_DEVICE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    hipStream_t strm = static_cast<hipStream_t>(stream);
    unsigned char* wsb = static_cast<unsigned char*>(ws);
    const DevicePlan dp = medusa_internal_device_plan(plan);

    GemmBatch g{};
    g.n_problems = 1;
    g.M = M;
    g.K = H;
    GemmProblem& p = g.p[0];
    p.W = w_lm;
    p.X = node_hidden;
    p.x_stride = H;
    p.N = V;
    p.tile_begin = 0;
    p.n_tiles = L.n_tiles;
    p.s = 1;
    p.part_val = reinterpret_cast<float*>(wsb + L.part_val);
    p.part_idx = reinterpret_cast<int32_t*>(wsb + L.part_idx);
    p.logits = logits;
    p.logits_ld = V;
    g.total_tiles = L.n_tiles;
    g.typ.inv_t = 1.0f / temperature;
    g.typ.part_z = reinterpret_cast<float*>(wsb + L.part_z);
    g.typ.part_s = reinterpret_cast<float*>(wsb + L.part_s);
    g.typ.parent = dp.parent;
    g.typ.node_tokens = node_tokens;
    g.typ.n_nodes = plan->n_nodes;
    g.typ.cand_logit = reinterpret_cast<float*>(wsb + L.cand_logit);
    hipError_t e = timed_gemm("verify_lmhead", dt, EPI_TYPICAL, g, strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);

    TypicalAccept ta{};
    ta.n_tiles = L.n_tiles;
    ta.part_val = p.part_val;
    ta.part_idx = p.part_idx;
    ta.part_z = g.typ.part_z;
    ta.part_s = g.typ.part_s;
    ta.cand_logit = g.typ.cand_logit;
    ta.node_tokens = node_tokens;
    ta.inv_t = g.typ.inv_t;
    ta.epsilon = epsilon;
    ta.delta = delta;
    ta.node_argmax = node_argmax ? node_argmax : reinterpret_cast<int32_t*>(wsb + L.node_arg);
    ta.node_max = reinterpret_cast<float*>(wsb + L.node_max);
    ta.node_z = reinterpret_cast<float*>(wsb + L.node_z);
    ta.node_tau = node_tau ? node_tau : reinterpret_cast<float*>(wsb + L.node_tau);
    ta.node_prob = node_prob;
    ta.accept_len = accept_len;
    ta.accept_nodes = accept_nodes;
    ta.accept_tokens = accept_tokens;
    prof_begin("verify_accept", strm);
    e = typical_accept_launch(dp, B, ta, strm);
    prof_end(strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    return MEDUSA_OK;
}

medusa_status medusa_rope(medusa_dtype dt, int M, int Hq, int Hkv, int d, const int32_t* positions,
                          float base, void* q, void* k, void* stream) {
    if (!positions || !q || !k) return MEDUSA_ERR_NULL;
    if (!dtype_ok(dt)) return MEDUSA_ERR_UNSUPPORTED;
    if (M < 1 || Hq < 1 || Hkv < 1 || d < 8 || d % 8 != 0 || d > 4096 ||
        (long long)M * (Hq + Hkv) * (d / 8) > (1LL << 31))
        return MEDUSA_ERR_SHAPE;
    if (!(base > 1.0f) || !std::isfinite(base)) return MEDUSA_ERR_SHAPE;
    const size_t align = dt == MEDUSA_BF16 ? 8 : 16;
    if (reinterpret_cast<uintptr_t>(q) % align || reinterpret_cast<uintptr_t>(k) % align)
        return MEDUSA_ERR_SHAPE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    RopeArgs a{};
    a.q = q;
    a.k = k;
    a.positions = positions;
    a.log2_base = std::log2((double)base);
    a.M = M;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.d = d;
    hipStream_t strm = static_cast<hipStream_t>(stream);
    prof_begin("rope", strm);
    hipError_t e = rope_launch(dt, a, strm);
    prof_end(strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    return MEDUSA_OK;
}

size_t medusa_hbm_probe_bytes(size_t bytes) { return (size_t)hbm_probe_bytes(bytes); }

medusa_status medusa_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink) return MEDUSA_ERR_NULL;
    if (hbm_probe_bytes(bytes) < 8192 || !aligned16(buf)) return MEDUSA_ERR_SHAPE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    hipError_t e = hbm_probe_launch(buf, bytes, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    return MEDUSA_OK;
}

medusa_status medusa_clock_probe(uint64_t* ticks, uint32_t* sink, void* stream) {
    if (!ticks || !sink) return MEDUSA_ERR_NULL;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    e = clock_probe_launch(reinterpret_cast<unsigned long long*>(ticks), sink, cus > 0 ? cus : 1,
                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    return MEDUSA_OK;
}

// ------------------------------------------------------------------ next round

medusa_status medusa_advance(const medusa_tree_plan* plan, medusa_dtype dt, int B, int H, int Hkv,
                             int d, int Lcap, const int32_t* accept_len,
                             const int32_t* accept_nodes, const int32_t* accept_tokens,
                             const void* k_tree, const void* v_tree, const void* node_hidden,
                             void* k_cache, void* v_cache, int32_t* prefix_lens, void* hidden_out,
                             int32_t* root_out, int32_t* overflow, void* stream) {
    if (!plan || !accept_len || !accept_nodes || !accept_tokens || !k_tree || !v_tree ||
        !node_hidden || !k_cache || !v_cache || !prefix_lens || !hidden_out || !root_out)
        return MEDUSA_ERR_NULL;
    if (!dtype_ok(dt)) return MEDUSA_ERR_UNSUPPORTED;
    const size_t es = esize(dt);
    if (B < 1 || B > 4096 || H < 1 || Hkv < 1 || d < 1 || Lcap < 1 || Lcap > (1 << 20))
        return MEDUSA_ERR_SHAPE;
    const size_t row_bytes = (size_t)Hkv * d * es;
    const size_t hidden_bytes = (size_t)H * es;
    if (row_bytes % 16 != 0 || hidden_bytes % 16 != 0) return MEDUSA_ERR_SHAPE;
    if (!aligned16(k_tree) || !aligned16(v_tree) || !aligned16(node_hidden) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(hidden_out))
        return MEDUSA_ERR_SHAPE;
    const int N = plan->n_nodes;
    // hidden_out is written while node_hidden is read
    const uintptr_t h0 = reinterpret_cast<uintptr_t>(hidden_out), h1 = h0 + (size_t)B * hidden_bytes;
    const uintptr_t n0 = reinterpret_cast<uintptr_t>(node_hidden), n1 = n0 + (size_t)B * N * hidden_bytes;
    if (h0 < n1 && n0 < h1) return MEDUSA_ERR_SHAPE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    AdvanceArgs a{};
    a.accept_len = accept_len;
    a.accept_nodes = accept_nodes;
    a.accept_tokens = accept_tokens;
    a.k_tree = k_tree;
    a.v_tree = v_tree;
    a.node_hidden = node_hidden;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.prefix_lens = prefix_lens;
    a.hidden_out = hidden_out;
    a.root_out = root_out;
    a.overflow = overflow;
    a.n_nodes = N;
    a.max_depth = plan->max_depth;
    a.Lcap = Lcap;
    a.row_bytes = (int)row_bytes;
    a.hidden_bytes = (int)hidden_bytes;
    hipStream_t strm = static_cast<hipStream_t>(stream);
    prof_begin("advance", strm);
    const hipError_t e = advance_launch(a, B, strm);
    prof_end(strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    return MEDUSA_OK;
}

// ------------------------------------------------------------------ one-layer verifier

namespace {

// Plans of the verifier's two projections (ksplit 0: direct store kernel).
PartialPlan qkv_plan(medusa_dtype dt, int M, int H, int Hq, int Hkv, int d) {
    const int Ns[3] = {Hq * d, Hkv * d, Hkv * d};
    return partial_plan(dt, M, H, Ns, 3);
}
PartialPlan out_plan(medusa_dtype dt, int M, int H, int Hq, int d) {
    return partial_plan(dt, M, Hq * d, &H, 1);
}
int qkv_ksplit(medusa_dtype dt, int M, int H, int Hq, int Hkv, int d) {
    return qkv_plan(dt, M, H, Hq, Hkv, d).ksplit;
}
int out_ksplit(medusa_dtype dt, int M, int H, int Hq, int d) {
    return out_plan(dt, M, H, Hq, d).ksplit;
}
// Weight-row tiles of one projection problem of width N.
int proxy_tiles(medusa_dtype dt, const PartialPlan& pl, int M, int N, int K) {
    if (pl.ksplit == 0) return n_tiles_for(dt, M, EPI_STORE, N, K);
    const int r = partial_tile_rows(pl);
    return (N + r - 1) / r;
}

}  // namespace

size_t medusa_proxy_workspace(medusa_dtype dt, int M, int H, int Hq, int Hkv, int d) {
    if (!dtype_ok(dt) || M < 1 || H < 1 || Hq < 1 || Hkv < 1 || d < 1) return 0;
    const size_t a = (size_t)qkv_ksplit(dt, M, H, Hq, Hkv, d) * M * (size_t)(Hq * d + 2 * Hkv * d);
    const size_t b = (size_t)out_ksplit(dt, M, H, Hq, d) * M * (size_t)H;
    return align256((a > b ? a : b) * sizeof(float)) + 256;
}

medusa_status medusa_proxy_qkv(medusa_dtype dt, int M, int H, int V, int Hq, int Hkv, int d,
                               const int32_t* tokens, const void* embed, const void* wq,
                               const void* wk, const void* wv, void* q, void* k, void* v,
                               void* ws, size_t ws_bytes, void* stream) {
    if (!tokens || !embed || !wq || !wk || !wv || !q || !k || !v) return MEDUSA_ERR_NULL;
    if (!dtype_ok(dt)) return MEDUSA_ERR_UNSUPPORTED;
    if (M < 1 || H < 32 || H > 16384 || H % 32 != 0 || V < 1 || Hq < 1 || Hkv < 1 || d < 1 ||
        (Hq * d) % 16 != 0 || (Hkv * d) % 16 != 0)
        return MEDUSA_ERR_SHAPE;
    if (!aligned16(embed) || !aligned16(wq) || !aligned16(wk) || !aligned16(wv))
        return MEDUSA_ERR_SHAPE;
    const PartialPlan pl = qkv_plan(dt, M, H, Hq, Hkv, d);
    const int ks = pl.ksplit;
    if (!ws || ws_bytes < medusa_proxy_workspace(dt, M, H, Hq, Hkv, d)) return MEDUSA_ERR_WORKSPACE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    GemmBatch g{};
    g.n_problems = 3;
    g.M = M;
    g.K = H;
    g.x_rows_bound = V;
    g.ksplit = ks > 0 ? ks : 1;
    const void* W[3] = {wq, wk, wv};
    void* O[3] = {q, k, v};
    const int Nn[3] = {Hq * d, Hkv * d, Hkv * d};
    int tiles = 0;
    float* part = static_cast<float*>(ws);
    for (int i = 0; i < 3; ++i) {
        GemmProblem& p = g.p[i];
        p.W = W[i];
        p.X = embed;
        p.x_rows = tokens;
        p.x_stride = H;
        p.N = Nn[i];
        p.tile_begin = tiles;
        p.n_tiles = proxy_tiles(dt, pl, M, Nn[i], H);
        tiles += p.n_tiles;
        p.out = O[i];
        p.ldo = Nn[i];
        p.part_val = part;
        part += (size_t)g.ksplit * M * Nn[i];
    }
    g.total_tiles = tiles;
    hipStream_t strm = static_cast<hipStream_t>(stream);
    hipError_t e;
    prof_begin("proxy_qkv", strm);
    e = ks > 0 ? gemm_store_partial_launch(dt, g, strm) : gemm_launch(dt, EPI_STORE, g, strm);
    prof_end(strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    return MEDUSA_OK;
}

medusa_status medusa_proxy_out(medusa_dtype dt, int M, int H, int V, int Hq, int d,
                               const int32_t* tokens, const void* embed, const void* o,
                               const void* wo, void* node_hidden, void* ws, size_t ws_bytes,
                               void* stream) {
    if (!tokens || !embed || !o || !wo || !node_hidden) return MEDUSA_ERR_NULL;
    if (!dtype_ok(dt)) return MEDUSA_ERR_UNSUPPORTED;
    if (M < 1 || H < 16 || H % 16 != 0 || V < 1 || Hq < 1 || d < 1 || (Hq * d) % 32 != 0)
        return MEDUSA_ERR_SHAPE;
    if (!aligned16(embed) || !aligned16(o) || !aligned16(wo)) return MEDUSA_ERR_SHAPE;
    const PartialPlan pl = out_plan(dt, M, H, Hq, d);
    const int ks = pl.ksplit;
    const size_t need = align256((size_t)(ks > 0 ? ks : 0) * M * (size_t)H * sizeof(float)) + 256;
    if (!ws || ws_bytes < need) return MEDUSA_ERR_WORKSPACE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    GemmBatch g{};
    g.n_problems = 1;
    g.M = M;
    g.K = Hq * d;
    g.res_rows_bound = V;
    g.ksplit = ks > 0 ? ks : 1;
    GemmProblem& p = g.p[0];
    p.W = wo;
    p.X = o;
    p.x_stride = (long long)Hq * d;
    p.N = H;
    p.tile_begin = 0;
    p.n_tiles = proxy_tiles(dt, pl, M, H, Hq * d);
    p.out = node_hidden;
    p.ldo = H;
    p.res = embed;
    p.res_rows = tokens;
    p.res_stride = H;
    p.part_val = static_cast<float*>(ws);
    g.total_tiles = p.n_tiles;
    hipStream_t strm = static_cast<hipStream_t>(stream);
    hipError_t e;
    prof_begin("proxy_out", strm);
    e = ks > 0 ? gemm_store_partial_launch(dt, g, strm) : gemm_launch(dt, EPI_STORE, g, strm);
    prof_end(strm);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    return MEDUSA_OK;
}

}  // extern "C"
