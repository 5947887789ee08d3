// Tree fill and greedy acceptance.
//
// Tree fill (glossary "Medusa Heads", section "Attention arborescente et acceptation"):
// node 0 carries the root token, a depth-d node with rank r carries head d's rank-r
// candidate; every head-d candidate appears under every depth-(d-1) node that the plan
// keeps, which is why the plan (parent/depth/rank) is static and only the tokens change.
//
// Acceptance (same section): a candidate is accepted when it equals the model's first
// choice at its parent; the longest accepted branch is kept and the deepest accepted
// node's own first choice is emitted after it.  Typical acceptance (same section, for
// sampling) keeps instead every candidate whose probability under its parent's
// distribution exceeds a threshold tied to that distribution's entropy; here
// tau = min(epsilon, delta * exp(-H)) at temperature T.
#include "common.hpp"
#include "internal.hpp"
#include "advance.hpp"

#include <limits.h>

namespace medusa {

namespace {

__global__ __launch_bounds__(256) void build_tree_kernel(DevicePlan plan, int K, int s_max,
                                                         const int32_t* __restrict__ root_ids,
                                                         const int32_t* __restrict__ topk_ids,
                                                         const int32_t* __restrict__ prefix_lens,
                                                         int32_t* __restrict__ node_tokens,
                                                         int32_t* __restrict__ position_ids) {
    const int b = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int N = plan.n_nodes;
    if (i >= N) return;
    const int d = plan.depth[i];
    const int tok = d == 0 ? root_ids[b]
                           : topk_ids[((long long)b * K + (d - 1)) * s_max + plan.rank[i]];
    node_tokens[(long long)b * N + i] = tok;
    if (position_ids) position_ids[(long long)b * N + i] = (prefix_lens ? prefix_lens[b] : 0) + d;
}

constexpr int kAcceptThreads = 1024;
constexpr int kMaxNodes = MEDUSA_MAX_NODES;
constexpr int kMergeThreads = 256;  // node merge: four nodes (one per wave) per workgroup
constexpr int kMergeBatch = 16;     // tile partials per lane in flight at once

struct NodeMerge {
    int n_rows;                 // B * n_nodes
    int n_tiles;
    const float* part_val;
    const int32_t* part_idx;
    const float* part_z;        // null: argmax only (greedy acceptance)
    const float* part_s;
    float inv_t, epsilon, delta;
    int32_t* node_argmax;       // [n_rows]
    float* node_max;            // [n_rows], typical only
    float* node_z;
    float* node_tau;
};

// Fold tiles t0, t0 + stride, ... (kMergeBatch of them, those below n) of one node's
// argmax partials into (bv, bi): every load is issued before the first comparison.
__device__ __forceinline__ void merge_batch(const float* pv, const int32_t* pi, int t0, int n,
                                            int stride, float& bv, int& bi) {
    float v[kMergeBatch];
    int id[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
        const int t = min(t0 + j * stride, n - 1);
        v[j] = pv[t];
        id[j] = pi[t];
    }
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
        if (t0 + j * stride < n && better(v[j], id[j], bv, bi)) { bv = v[j]; bi = id[j]; }
}

// The kept branch: the deepest accepted node, the lowest index among equals (atomicMax on
// (depth, -index)); its path root-first, the candidates on it, then the node's argmax.
// s_acc must be final and visible to every thread; s_best starts at 0.
__device__ __forceinline__ void emit_branch(const DevicePlan& plan, int b,
                                            const unsigned char* s_acc, const int* s_arg,
                                            const int32_t* tok, int& s_best, int32_t* accept_len,
                                            int32_t* accept_nodes, int32_t* accept_tokens) {
    const int N = plan.n_nodes;
    const int D = plan.max_depth;
    for (int i = threadIdx.x; i < N; i += kAcceptThreads)
        if (s_acc[i]) atomicMax(&s_best, (plan.depth[i] << 16) | (0xFFFF - i));
    __syncthreads();
    if (threadIdx.x == 0) {
        const int best = 0xFFFF - (s_best & 0xFFFF);
        const int a = plan.depth[best];
        accept_len[b] = a;
        int32_t* an = accept_nodes + (long long)b * (D + 1);
        int32_t* at = accept_tokens + (long long)b * (D + 1);
        for (int j = a + 1; j <= D; ++j) { an[j] = -1; at[j] = -1; }
        int node = best;
        for (int j = a; j >= 0; --j) {
            an[j] = node;
            if (j >= 1) at[j - 1] = tok[node];
            node = plan.parent[node];
        }
        at[a] = s_arg[best];
    }
}

// Per-node merge of the lm_head tile partials, one wave per node over many workgroups so
// the partials stream through many CUs: the node's argmax and, for typical acceptance,
// its maximum, softmax normaliser and threshold.  With y = (tile max - node max) / T, the
// tiles' sums combine as Z = sum z e^y and S = sum e^y (s + z y), and H = ln Z - S / Z.
__global__ __launch_bounds__(kMergeThreads) void node_merge_kernel(NodeMerge a) {
    constexpr float kLog2e = 1.4426950408889634f;
    const int row = blockIdx.x * (kMergeThreads / kWave) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= a.n_rows) return;            // a whole wave: this kernel has no block barrier
    const int nt = a.n_tiles;
    const long long base = (long long)row * nt;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int t0 = lane; t0 < nt; t0 += kMergeBatch * kWave)
        merge_batch(a.part_val + base, a.part_idx + base, t0, nt, kWave, bv, bi);
    wave_best(bv, bi);
    if (!a.part_z) {
        if (lane == 0) a.node_argmax[row] = bi;
        return;
    }
    float z = 0.f, sx = 0.f;
    for (int t0 = lane; t0 < nt; t0 += kMergeBatch * kWave) {
        float pv[kMergeBatch], pz[kMergeBatch], ps[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {     // every load before the first use
            const int t = min(t0 + j * kWave, nt - 1);
            pv[j] = a.part_val[base + t];
            pz[j] = a.part_z[base + t];
            ps[j] = a.part_s[base + t];
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            if (t0 + j * kWave >= nt) continue;
            const float y = (pv[j] - bv) * a.inv_t;
            const float g = __builtin_amdgcn_exp2f(y * kLog2e);
            z += g * pz[j];
            sx += g * (ps[j] + pz[j] * y);
        }
    }
    z = wave_sum_dpp(z);
    sx = wave_sum_dpp(sx);
    if (lane == 0) {
        const float H = logf(z) - sx / z;
        a.node_argmax[row] = bi;
        a.node_max[row] = bv;
        a.node_z[row] = z;
        a.node_tau[row] = fminf(a.epsilon, a.delta * expf(-H));
    }
}

// Greedy walk, one workgroup per sequence: a node is accepted when its parent is and its
// token is the parent's argmax.
__global__ __launch_bounds__(kAcceptThreads) void accept_walk_kernel(
    DevicePlan plan, const int32_t* __restrict__ node_argmax,
    const int32_t* __restrict__ node_tokens, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ accept_nodes, int32_t* __restrict__ accept_tokens) {
    __shared__ int s_arg[kMaxNodes];
    __shared__ unsigned char s_acc[kMaxNodes];
    __shared__ int s_best;
    const int b = blockIdx.x;
    const int N = plan.n_nodes;
    const int D = plan.max_depth;
    for (int i = threadIdx.x; i < N; i += kAcceptThreads) {
        s_arg[i] = node_argmax[(long long)b * N + i];
        s_acc[i] = i == 0;
    }
    if (threadIdx.x == 0) s_best = 0;
    __syncthreads();
    const int32_t* tok = node_tokens + (long long)b * N;
    for (int d = 1; d <= D; ++d) {
        for (int i = threadIdx.x; i < N; i += kAcceptThreads) {
            if (plan.depth[i] != d) continue;
            const int p = plan.parent[i];
            s_acc[i] = s_acc[p] && tok[i] == s_arg[p];
        }
        __syncthreads();
    }
    emit_branch(plan, b, s_acc, s_arg, tok, s_best, accept_len, accept_nodes, accept_tokens);
}

// Typical walk, one workgroup per sequence: each candidate's probability under its
// parent's distribution, p = e^((logit - max) / T) / Z, and a node is accepted when its
// parent is and p exceeds the parent's threshold.
__global__ __launch_bounds__(kAcceptThreads) void typical_walk_kernel(DevicePlan plan,
                                                                      TypicalAccept a) {
    __shared__ int s_arg[kMaxNodes];
    __shared__ float s_tau[kMaxNodes];
    __shared__ float s_prob[kMaxNodes];
    __shared__ unsigned char s_acc[kMaxNodes];
    __shared__ int s_best;
    constexpr float kLog2e = 1.4426950408889634f;
    const int b = blockIdx.x;
    const int N = plan.n_nodes;
    const int D = plan.max_depth;
    const long long o = (long long)b * N;
    for (int c = threadIdx.x; c < N; c += kAcceptThreads) {
        s_arg[c] = a.node_argmax[o + c];
        s_tau[c] = a.node_tau[o + c];
        float p = 1.f;
        if (c > 0) {
            const int par = plan.parent[c];
            const float y = (a.cand_logit[o + c] - a.node_max[o + par]) * a.inv_t;
            p = __builtin_amdgcn_exp2f(y * kLog2e) / a.node_z[o + par];
        }
        s_prob[c] = p;
        s_acc[c] = c == 0;
        if (a.node_prob) a.node_prob[o + c] = p;
    }
    if (threadIdx.x == 0) s_best = 0;
    __syncthreads();
    for (int d = 1; d <= D; ++d) {
        for (int i = threadIdx.x; i < N; i += kAcceptThreads) {
            if (plan.depth[i] != d) continue;
            const int par = plan.parent[i];
            s_acc[i] = s_acc[par] && s_prob[i] > s_tau[par];
        }
        __syncthreads();
    }
    emit_branch(plan, b, s_acc, s_arg, a.node_tokens + o, s_best, a.accept_len, a.accept_nodes,
                a.accept_tokens);
}

// Next round (same section: the longest accepted branch is kept and its last hidden state
// feeds the heads next time): the branch's tree K/V rows join the cache after the prefix,
// the deepest accepted node's hidden state and bonus token become the next h and root.
// One workgroup per sequence; every row moves as 16-byte vectors.  All threads read the
// old length before thread 0 replaces it.
__global__ __launch_bounds__(256) void advance_kernel(AdvanceArgs a) {
    const int b = blockIdx.x;
    const int D1 = a.max_depth + 1;
    const int L = a.prefix_lens[b];
    const int acc = min(max(a.accept_len[b], 0), a.max_depth);
    const bool fits = L >= 0 && L + acc + 1 <= a.Lcap;
    const int32_t* nodes = a.accept_nodes + (long long)b * D1;
    auto node_at = [&](int j) { return min(max(nodes[j], 0), a.n_nodes - 1); };
    if (fits) {
        const int vpr = a.row_bytes / 16;                     // vectors per K/V row
        const int total = (acc + 1) * vpr;
        for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
            const int j = idx / vpr;
            const int c = idx - j * vpr;
            const long long src = ((long long)b * a.n_nodes + node_at(j)) * vpr + c;
            const long long dst = ((long long)b * a.Lcap + L + j) * vpr + c;
            reinterpret_cast<u32x4*>(a.k_cache)[dst] = reinterpret_cast<const u32x4*>(a.k_tree)[src];
            reinterpret_cast<u32x4*>(a.v_cache)[dst] = reinterpret_cast<const u32x4*>(a.v_tree)[src];
        }
        const int hv = a.hidden_bytes / 16;
        const long long hsrc = ((long long)b * a.n_nodes + node_at(acc)) * hv;
        for (int c = threadIdx.x; c < hv; c += blockDim.x)
            reinterpret_cast<u32x4*>(a.hidden_out)[(long long)b * hv + c] =
                reinterpret_cast<const u32x4*>(a.node_hidden)[hsrc + c];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        if (fits) {
            a.prefix_lens[b] = L + acc + 1;
            a.root_out[b] = a.accept_tokens[(long long)b * D1 + acc];
        }
        if (a.overflow) a.overflow[b] = fits ? 0 : 1;
    }
}

}  // namespace

hipError_t typical_accept_launch(const DevicePlan& plan, int B, const TypicalAccept& a,
                                 hipStream_t stream) {
    NodeMerge m{};
    m.n_rows = B * plan.n_nodes;
    m.n_tiles = a.n_tiles;
    m.part_val = a.part_val;
    m.part_idx = a.part_idx;
    m.part_z = a.part_z;
    m.part_s = a.part_s;
    m.inv_t = a.inv_t;
    m.epsilon = a.epsilon;
    m.delta = a.delta;
    m.node_argmax = a.node_argmax;
    m.node_max = a.node_max;
    m.node_z = a.node_z;
    m.node_tau = a.node_tau;
    const int per = kMergeThreads / kWave;
    hipLaunchKernelGGL(node_merge_kernel, dim3((m.n_rows + per - 1) / per), dim3(kMergeThreads), 0,
                       stream, m);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(typical_walk_kernel, dim3(B), dim3(kAcceptThreads), 0, stream, plan, a);
    return hipGetLastError();
}

hipError_t advance_launch(const AdvanceArgs& args, int B, hipStream_t stream) {
    hipLaunchKernelGGL(advance_kernel, dim3(B), dim3(256), 0, stream, args);
    return hipGetLastError();
}


hipError_t build_tree_launch(const DevicePlan& plan, int B, int K, int s_max,
                             const int32_t* root_ids, const int32_t* topk_ids,
                             const int32_t* prefix_lens, int32_t* node_tokens,
                             int32_t* position_ids, hipStream_t stream) {
    dim3 grid((plan.n_nodes + 255) / 256, B);
    hipLaunchKernelGGL(build_tree_kernel, grid, dim3(256), 0, stream, plan, K, s_max, root_ids,
                       topk_ids, prefix_lens, node_tokens, position_ids);
    return hipGetLastError();
}

hipError_t accept_launch(const DevicePlan& plan, int B, int n_tiles, const float* part_val,
                         const int32_t* part_idx, const int32_t* node_tokens,
                         int32_t* node_argmax, int32_t* accept_len, int32_t* accept_nodes,
                         int32_t* accept_tokens, hipStream_t stream) {
    NodeMerge m{};
    m.n_rows = B * plan.n_nodes;
    m.n_tiles = n_tiles;
    m.part_val = part_val;
    m.part_idx = part_idx;
    m.node_argmax = node_argmax;
    const int per = kMergeThreads / kWave;
    hipLaunchKernelGGL(node_merge_kernel, dim3((m.n_rows + per - 1) / per), dim3(kMergeThreads), 0,
                       stream, m);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(accept_walk_kernel, dim3(B), dim3(kAcceptThreads), 0, stream, plan,
                       node_argmax, node_tokens, accept_len, accept_nodes, accept_tokens);
    return hipGetLastError();
}

}  // namespace medusa
