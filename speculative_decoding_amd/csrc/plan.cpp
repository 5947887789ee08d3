// Candidate-tree plans (host side).
//
// Glossary "Medusa Heads", section "Attention arborescente et acceptation": the heads'
// best hypotheses combine as a Cartesian product into continuations that share prefixes
// and form a tree; a sparse tree of the most accurate combinations (64 nodes) beats a
// dense one (256 nodes).  A node is a rank tuple (i_1..i_d); node 0 (the empty tuple) is
// the root.  Nodes are kept breadth first (depth, then tuple ascending), which puts every
// parent before its children and gives siblings contiguous ranks.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <new>
#include <vector>

#include "plan_impl.hpp"

namespace {

using Tuple = std::vector<int32_t>;

bool tuple_less(const Tuple& a, const Tuple& b) {
    if (a.size() != b.size()) return a.size() < b.size();
    return a < b;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

medusa_status finish(std::vector<Tuple> tuples, medusa_tree_plan** out) {
    if (tuples.size() + 1 > (size_t)MEDUSA_MAX_NODES) return MEDUSA_ERR_SHAPE;
    std::map<Tuple, int> present;
    for (const Tuple& t : tuples) {
        if (t.empty()) return MEDUSA_ERR_TREE;
        for (int32_t r : t)
            if (r < 0 || r >= MEDUSA_MAX_TOPK) return MEDUSA_ERR_TREE;
        if (!present.emplace(t, 0).second) return MEDUSA_ERR_TREE;      // duplicate
    }
    for (const Tuple& t : tuples) {
        if (t.size() > 1) {
            Tuple p(t.begin(), t.end() - 1);
            if (!present.count(p)) return MEDUSA_ERR_TREE;                // not prefix-closed
        }
    }
    std::sort(tuples.begin(), tuples.end(), tuple_less);
    medusa_tree_plan* plan = new (std::nothrow) medusa_tree_plan();
    if (!plan) return MEDUSA_ERR_SHAPE;
    const int N = (int)tuples.size() + 1;
    plan->n_nodes = N;
    plan->mask_words = (N + 63) / 64;
    plan->parent.assign(N, -1);
    plan->depth.assign(N, 0);
    plan->rank.assign(N, -1);
    plan->mask.assign((size_t)N * plan->mask_words, 0ull);
    std::map<Tuple, int> index;
    index[Tuple()] = 0;
    for (int i = 1; i < N; ++i) index[tuples[i - 1]] = i;
    plan->max_depth = 0;
    for (int i = 0; i < N; ++i) {
        const Tuple t = i == 0 ? Tuple() : tuples[i - 1];
        plan->depth[i] = (int32_t)t.size();
        plan->max_depth = std::max(plan->max_depth, (int)t.size());
        if (!t.empty()) {
            plan->parent[i] = index[Tuple(t.begin(), t.end() - 1)];
            plan->rank[i] = t.back();
        }
        for (size_t d = 0; d <= t.size(); ++d) {
            const int j = index[Tuple(t.begin(), t.begin() + d)];
            plan->mask[(size_t)i * plan->mask_words + j / 64] |= 1ull << (j % 64);
        }
    }
    // device image: parent | depth | rank | mask, each 256-byte aligned
    plan->off_depth = align256(sizeof(int32_t) * N);
    plan->off_rank = plan->off_depth + align256(sizeof(int32_t) * N);
    plan->off_mask = plan->off_rank + align256(sizeof(int32_t) * N);
    plan->image_bytes = plan->off_mask + align256(sizeof(uint64_t) * plan->mask.size());
    plan->image.assign(plan->image_bytes, 0);
    std::memcpy(plan->image.data(), plan->parent.data(), sizeof(int32_t) * N);
    std::memcpy(plan->image.data() + plan->off_depth, plan->depth.data(), sizeof(int32_t) * N);
    std::memcpy(plan->image.data() + plan->off_rank, plan->rank.data(), sizeof(int32_t) * N);
    std::memcpy(plan->image.data() + plan->off_mask, plan->mask.data(),
                sizeof(uint64_t) * plan->mask.size());
    *out = plan;
    return MEDUSA_OK;
}

// All rank tuples of the Cartesian product of tree_s[0..d) for d = 1..depth, or an error
// when there would be more than `limit`.
medusa_status enumerate(const int32_t* tree_s, int depth, size_t limit, std::vector<Tuple>* out) {
    size_t total = 0, level = 1;
    for (int d = 0; d < depth; ++d) {
        if (tree_s[d] < 1 || tree_s[d] > MEDUSA_MAX_TOPK) return MEDUSA_ERR_SHAPE;
        level *= (size_t)tree_s[d];
        total += level;
        if (total > limit) return MEDUSA_ERR_SHAPE;
    }
    out->clear();
    out->reserve(total);
    std::vector<Tuple> frontier{Tuple()};
    for (int d = 0; d < depth; ++d) {
        std::vector<Tuple> next;
        next.reserve(frontier.size() * tree_s[d]);
        for (const Tuple& t : frontier)
            for (int32_t r = 0; r < tree_s[d]; ++r) {
                Tuple c = t;
                c.push_back(r);
                next.push_back(c);
            }
        out->insert(out->end(), next.begin(), next.end());
        frontier.swap(next);
    }
    return MEDUSA_OK;
}

}  // namespace

extern "C" {

medusa_status medusa_tree_plan_create(const int32_t* paths, int n_paths, int max_depth,
                                      medusa_tree_plan** out) {
    if (!out || (n_paths > 0 && !paths)) return MEDUSA_ERR_NULL;
    if (n_paths < 0 || max_depth < 0 || (n_paths > 0 && max_depth < 1)) return MEDUSA_ERR_SHAPE;
    if (n_paths + 1 > MEDUSA_MAX_NODES) return MEDUSA_ERR_SHAPE;
    std::vector<Tuple> tuples;
    tuples.reserve(n_paths);
    for (int p = 0; p < n_paths; ++p) {
        Tuple t;
        bool ended = false;
        for (int d = 0; d < max_depth; ++d) {
            const int32_t r = paths[(size_t)p * max_depth + d];
            if (r < 0) {
                ended = true;
                continue;
            }
            if (ended) return MEDUSA_ERR_TREE;     // a rank after the padding
            t.push_back(r);
        }
        tuples.push_back(t);
    }
    return finish(std::move(tuples), out);
}

medusa_status medusa_tree_plan_full(const int32_t* tree_s, int depth, medusa_tree_plan** out) {
    if (!out || (depth > 0 && !tree_s)) return MEDUSA_ERR_NULL;
    if (depth < 0) return MEDUSA_ERR_SHAPE;
    std::vector<Tuple> tuples;
    medusa_status st = enumerate(tree_s, depth, MEDUSA_MAX_NODES - 1, &tuples);
    if (st != MEDUSA_OK) return st;
    return finish(std::move(tuples), out);
}

medusa_status medusa_tree_plan_from_accuracy(const double* acc, int acc_stride,
                                             const int32_t* tree_s, int depth, int n_nodes,
                                             medusa_tree_plan** out) {
    if (!out || !acc || !tree_s) return MEDUSA_ERR_NULL;
    if (depth < 1 || n_nodes < 1 || n_nodes > MEDUSA_MAX_NODES) return MEDUSA_ERR_SHAPE;
    for (int d = 0; d < depth; ++d)
        if (tree_s[d] < 1 || tree_s[d] > acc_stride) return MEDUSA_ERR_SHAPE;
    std::vector<Tuple> cands;
    medusa_status st = enumerate(tree_s, depth, size_t(1) << 22, &cands);
    if (st != MEDUSA_OK) return st;
    if ((size_t)n_nodes - 1 > cands.size()) return MEDUSA_ERR_SHAPE;
    std::vector<double> score(cands.size());
    for (size_t c = 0; c < cands.size(); ++c) {
        double p = 1.0;
        for (size_t d = 0; d < cands[c].size(); ++d) p *= acc[d * (size_t)acc_stride + cands[c][d]];
        score[c] = p;
    }
    std::vector<size_t> order(cands.size());
    for (size_t c = 0; c < order.size(); ++c) order[c] = c;
    std::sort(order.begin(), order.end(), [&](size_t a, size_t b) {
        if (score[a] != score[b]) return score[a] > score[b];
        return tuple_less(cands[a], cands[b]);
    });
    std::vector<Tuple> keep;
    keep.reserve(n_nodes - 1);
    for (int i = 0; i < n_nodes - 1; ++i) keep.push_back(cands[order[i]]);
    return finish(std::move(keep), out);
}

medusa_status medusa_tree_plan_expected_accept(const medusa_tree_plan* plan, const double* acc,
                                               int acc_stride, int acc_rows, double* out) {
    if (!plan || !acc || !out) return MEDUSA_ERR_NULL;
    if (acc_rows < plan->max_depth || acc_stride < 1) return MEDUSA_ERR_SHAPE;
    // nodes are breadth first, so a parent's path probability is known before its children's
    std::vector<double> path(plan->n_nodes, 1.0);
    double sum = 0.0;
    for (int i = 1; i < plan->n_nodes; ++i) {
        const int d = plan->depth[i], r = plan->rank[i];
        if (r >= acc_stride) return MEDUSA_ERR_SHAPE;
        path[i] = path[plan->parent[i]] * acc[(size_t)(d - 1) * acc_stride + r];
        sum += path[i];
    }
    *out = sum;
    return MEDUSA_OK;
}

medusa_status medusa_tree_plan_info(const medusa_tree_plan* plan, int* n_nodes, int* max_depth,
                                    int* mask_words) {
    if (!plan) return MEDUSA_ERR_NULL;
    if (n_nodes) *n_nodes = plan->n_nodes;
    if (max_depth) *max_depth = plan->max_depth;
    if (mask_words) *mask_words = plan->mask_words;
    return MEDUSA_OK;
}

medusa_status medusa_tree_plan_arrays(const medusa_tree_plan* plan, int32_t* parent,
                                      int32_t* depth, int32_t* rank, uint64_t* mask) {
    if (!plan) return MEDUSA_ERR_NULL;
    const size_t N = plan->n_nodes;
    if (parent) std::memcpy(parent, plan->parent.data(), N * sizeof(int32_t));
    if (depth) std::memcpy(depth, plan->depth.data(), N * sizeof(int32_t));
    if (rank) std::memcpy(rank, plan->rank.data(), N * sizeof(int32_t));
    if (mask) std::memcpy(mask, plan->mask.data(), plan->mask.size() * sizeof(uint64_t));
    return MEDUSA_OK;
}

size_t medusa_tree_plan_device_bytes(const medusa_tree_plan* plan) {
    return plan ? plan->image_bytes : 0;
}

medusa_status medusa_tree_plan_upload(medusa_tree_plan* plan, void* device_buf, size_t bytes,
                                      void* stream) {
    if (!plan || !device_buf) return MEDUSA_ERR_NULL;
    if (bytes < plan->image_bytes) return MEDUSA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(device_buf) & 255) != 0) return MEDUSA_ERR_SHAPE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(device_buf, plan->image.data(), plan->image_bytes,
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    plan->dev = static_cast<unsigned char*>(device_buf);
    return MEDUSA_OK;
}

void medusa_tree_plan_destroy(medusa_tree_plan* plan) { delete plan; }

}  // extern "C"
