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
constexpr int kMergeBatch = 16;     // tile partials per lane in flight at once

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

// One workgroup per sequence: merge the lm_head argmax partials of every node, then walk
// the tree level by level.
__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(
    DevicePlan plan, int n_tiles, const float* __restrict__ part_val,
    const int32_t* __restrict__ part_idx, const int32_t* __restrict__ node_tokens,
    int32_t* __restrict__ node_argmax, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ accept_nodes, int32_t* __restrict__ accept_tokens) {
    __shared__ int s_arg[kMaxNodes];
    __shared__ unsigned char s_acc[kMaxNodes];
    __shared__ int s_best;
    const int b = blockIdx.x;
    const int N = plan.n_nodes;
    const int D = plan.max_depth;
    // 16 lanes per node: each lane scans a strided share of the node's tile partials,
    // kMergeBatch loads in flight at a time, then the 16 lanes reduce.
    constexpr int kPerNode = 16;
    for (int i0 = 0; i0 < N; i0 += kAcceptThreads / kPerNode) {
        const int i = i0 + threadIdx.x / kPerNode;
        const int sub = threadIdx.x % kPerNode;
        float bv = -INFINITY;
        int bi = INT_MAX;
        if (i < N) {
            const float* pv = part_val + ((long long)b * N + i) * n_tiles;
            const int32_t* pi = part_idx + ((long long)b * N + i) * n_tiles;
            for (int t0 = sub; t0 < n_tiles; t0 += kMergeBatch * kPerNode)
                merge_batch(pv, pi, t0, n_tiles, kPerNode, bv, bi);
        }
        row_best(bv, bi);     // the 16 lanes of a node form one DPP row
        if (sub == 0 && i < N) {
            s_arg[i] = bi;
            if (node_argmax) node_argmax[(long long)b * N + i] = bi;
        }
    }
    for (int i = threadIdx.x; i < N; i += kAcceptThreads) s_acc[i] = i == 0;
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

// Per node: argmax, the softmax normaliser and the entropy merged over the lm_head tiles,
// and the threshold; per candidate: its probability under the parent's distribution; then
// the level walk.  One workgroup per sequence, 16 lanes per node for the merges.
__global__ __launch_bounds__(kAcceptThreads) void typical_accept_kernel(DevicePlan plan,
                                                                        TypicalAccept a) {
    __shared__ int s_arg[kMaxNodes];
    __shared__ float s_max[kMaxNodes];
    __shared__ float s_z[kMaxNodes];
    __shared__ float s_tau[kMaxNodes];
    __shared__ float s_prob[kMaxNodes];
    __shared__ unsigned char s_acc[kMaxNodes];
    __shared__ int s_best;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr int kPerNode = 16;
    const int b = blockIdx.x;
    const int N = plan.n_nodes;
    const int D = plan.max_depth;
    const int nt = a.n_tiles;
    for (int i0 = 0; i0 < N; i0 += kAcceptThreads / kPerNode) {
        const int i = i0 + threadIdx.x / kPerNode;
        const int sub = threadIdx.x % kPerNode;
        const long long base = ((long long)b * N + min(i, N - 1)) * nt;
        float bv = -INFINITY;
        int bi = INT_MAX;
        for (int t0 = sub; t0 < nt; t0 += kMergeBatch * kPerNode)
            merge_batch(a.part_val + base, a.part_idx + base, t0, nt, kPerNode, bv, bi);
        row_best(bv, bi);       // every lane of the node's row: the maximum and its id
        // the tiles' sums rescaled to the node's maximum: with y = (tile max - max) / T,
        // Z = sum z e^y and S = sum e^y (s + z y), so that H = ln Z - S / Z; the loads of
        // a batch are all issued before the first is used
        float z = 0.f, sx = 0.f;
        for (int t0 = sub; t0 < nt; t0 += kMergeBatch * kPerNode) {
            float pv[kMergeBatch], pz[kMergeBatch], ps[kMergeBatch];
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
                const int t = min(t0 + j * kPerNode, nt - 1);
                pv[j] = a.part_val[base + t];
                pz[j] = a.part_z[base + t];
                ps[j] = a.part_s[base + t];
            }
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
                if (t0 + j * kPerNode >= nt) continue;
                const float y = (pv[j] - bv) * a.inv_t;
                const float g = __builtin_amdgcn_exp2f(y * kLog2e);
                z += g * pz[j];
                sx += g * (ps[j] + pz[j] * y);
            }
        }
        z = row_sum16(z);
        sx = row_sum16(sx);
        if (sub == 0 && i < N) {
            const float H = logf(z) - sx / z;
            const float tau = fminf(a.epsilon, a.delta * expf(-H));
            s_arg[i] = bi;
            s_max[i] = bv;
            s_z[i] = z;
            s_tau[i] = tau;
            if (a.node_argmax) a.node_argmax[(long long)b * N + i] = bi;
            if (a.node_tau) a.node_tau[(long long)b * N + i] = tau;
        }
    }
    if (threadIdx.x == 0) s_best = 0;
    __syncthreads();
    for (int c = threadIdx.x; c < N; c += kAcceptThreads) {
        float p = 1.f;
        if (c > 0) {
            const int par = plan.parent[c];
            const float y = (a.cand_logit[(long long)b * N + c] - s_max[par]) * a.inv_t;
            p = __builtin_amdgcn_exp2f(y * kLog2e) / s_z[par];
        }
        s_prob[c] = p;
        s_acc[c] = c == 0;
        if (a.node_prob) a.node_prob[(long long)b * N + c] = p;
    }
    __syncthreads();
    for (int d = 1; d <= D; ++d) {
        for (int i = threadIdx.x; i < N; i += kAcceptThreads) {
            if (plan.depth[i] != d) continue;
            const int par = plan.parent[i];
            s_acc[i] = s_acc[par] && s_prob[i] > s_tau[par];
        }
        __syncthreads();
    }
    emit_branch(plan, b, s_acc, s_arg, a.node_tokens + (long long)b * N, s_best, a.accept_len,
                a.accept_nodes, a.accept_tokens);
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
    hipLaunchKernelGGL(typical_accept_kernel, dim3(B), dim3(kAcceptThreads), 0, stream, plan, a);
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
    hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(kAcceptThreads), 0, stream, plan, n_tiles,
                       part_val, part_idx, node_tokens, node_argmax, accept_len, accept_nodes,
                       accept_tokens);
    return hipGetLastError();
}

}  // namespace medusa
