// Internal interfaces between the C-ABI layer (api.cpp) and the kernels (*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/medusa.h"

namespace medusa {

// ------------------------------------------------------------------ skinny GEMM
// Y[m, n] = sum_k X[m, k] * W[n, k] for up to kMaxProblems independent problems that
// share M and K, in one launch.  W streams from HBM once; X rows are staged in LDS.
constexpr int kMaxProblems = 9;

enum Epilogue : int {
    EPI_STORE = 0,   // out[m*ldo + n] = rnd(silu?(acc + bias[n]) + residual[m][n])
    EPI_TOPS = 1,    // per row m: the tile's top-s (value desc, id asc) -> partials
    EPI_ARGMAX = 2,  // per row m: the tile's best (value, id) -> partials
    EPI_PARTIAL = 3, // fp32 partial sums of one contraction slice -> part_val[slice][m][n]
    EPI_TYPICAL = 4, // EPI_ARGMAX plus the tile's softmax sums and the tree candidates' logits
};

// Extra outputs of the EPI_TYPICAL epilogue (lm_head over the tree nodes; row m = b*n_nodes+i).
// With x = (logit - tile max) / T per vocabulary entry of the tile:
//   part_z[m][tile] = sum exp(x),  part_s[m][tile] = sum exp(x) * x
// and for every non-root node c of sequence b, the logit of c's token in its parent's row:
//   cand_logit[b*n_nodes + c] = logit[b*n_nodes + parent[c]][node_tokens[b*n_nodes + c]].
struct TypicalEpi {
    float inv_t;                 // 1 / temperature
    float* part_z;               // [M, n_tiles]
    float* part_s;
    const int32_t* parent;       // the plan's parents (device)
    const int32_t* node_tokens;  // [B, n_nodes]
    int n_nodes;
    float* cand_logit;           // [B, n_nodes]; root entries untouched
};

struct GemmProblem {
    const void* W;            // [N, K]
    const void* X;            // row m at X + (x_rows ? x_rows[m] : m) * x_stride
    const int32_t* x_rows;    // optional row gather (ids outside [0, x_rows_bound) read zeros)
    long long x_stride;       // elements
    int N;
    int tile_begin;           // first flattened tile of this problem
    int n_tiles;
    // EPI_STORE
    void* out;                // element type T
    long long ldo;
    const void* bias;         // [N] T or null
    int silu;                 // apply SiLU after the bias
    const void* res;          // residual rows (T) or null
    const int32_t* res_rows;  // optional residual gather
    long long res_stride;
    // EPI_TOPS / EPI_ARGMAX
    int s;                    // candidates kept per tile (1 for EPI_ARGMAX)
    float* logits;            // optional fp32 [M, N] with row stride logits_ld
    long long logits_ld;
    float* part_val;          // [M, n_tiles, s]
    int32_t* part_idx;
};

struct GemmBatch {
    GemmProblem p[kMaxProblems];
    int n_problems;
    int total_tiles;
    int M;
    int K;
    int KC;                   // contraction chunk staged in LDS per pass
    int x_rows_bound;
    int res_rows_bound;
    int ksplit;               // contraction slices (EPI_PARTIAL); 1 otherwise
    TypicalEpi typ;           // EPI_TYPICAL only
};

// Rows of W per workgroup (one tile) for a given configuration; N is the problem's width
// (the argmax and typical tiles at up to 64 rows are smaller for a small vocabulary).
int gemm_rows_per_tile(medusa_dtype dt, int M, int epi, int K, int N);
// Fills KC and launches.  Returns hipSuccess or the launch error.
hipError_t gemm_launch(medusa_dtype dt, int epi, GemmBatch& batch, hipStream_t stream);

// Store GEMMs with many input rows (the verifier's projections) run as contraction slices
// (EPI_PARTIAL) plus a finalize pass that sums the slices in order and applies the store
// epilogue.  partial_plan() picks the slice count and the kernel shape from the problem
// sizes alone (the same answer for the workspace query and the launch); ksplit == 0 means
// no split (the direct store kernel).  The caller points each problem's part_val at
// ksplit*M*N floats and sets batch.ksplit to the plan's.
struct PartialPlan {
    int ksplit;     // contraction slices; 0: not applicable
    int waves;      // waves per workgroup of the one-workgroup-per-CU kernel; 0: single-wave kernel
    int tile;       // 1: the 256 x 256 tiled kernel writes the slices (many input rows)
};
PartialPlan partial_plan(medusa_dtype dt, int M, int K, const int* Ns, int n);
// Weight rows per tile of a plan's slice kernel (problem tiles: ceil(N / this)).
int partial_tile_rows(const PartialPlan& pl);
hipError_t gemm_store_partial_launch(medusa_dtype dt, GemmBatch& batch, hipStream_t stream);

// ------------------------------------------------------------------ top-s merge
struct MergeProblem {
    const float* part_val;    // [M, n_tiles, s]
    const int32_t* part_idx;
    int n_tiles;
    int s;
    int32_t* out_ids;         // row m at out_ids + m * out_ld ; s_pad entries written
    float* out_vals;          // may be null
    long long out_ld;
    int s_pad;                // entries written per row (>= s); the rest get -1 / 0
};
struct MergeBatch {
    MergeProblem p[kMaxProblems];
    int n_problems;
    int M;
};
hipError_t topk_merge_launch(const MergeBatch& batch, hipStream_t stream);

// ------------------------------------------------------------------ tree
struct DevicePlan {
    const int32_t* parent;
    const int32_t* depth;
    const int32_t* rank;
    const uint64_t* mask;
    int n_nodes;
    int max_depth;
    int mask_words;
};
hipError_t build_tree_launch(const DevicePlan& plan, int B, int K, int s_max,
                             const int32_t* root_ids, const int32_t* topk_ids,
                             const int32_t* prefix_lens, int32_t* node_tokens,
                             int32_t* position_ids, hipStream_t stream);
// Greedy acceptance from the EPI_ARGMAX partials: a per-node merge over many workgroups
// (node_argmax [B, n_nodes], required), then the level walk, one workgroup per sequence.
hipError_t accept_launch(const DevicePlan& plan, int B, int n_tiles, const float* part_val,
                         const int32_t* part_idx, const int32_t* node_tokens,
                         int32_t* node_argmax, int32_t* accept_len, int32_t* accept_nodes,
                         int32_t* accept_tokens, hipStream_t stream);
// Typical acceptance from the EPI_TYPICAL partials: per node the argmax, the softmax
// normaliser and entropy (merged over the tiles), the threshold min(epsilon, delta*exp(-H))
// and each candidate's probability under its parent's distribution; then the branch walk.
struct TypicalAccept {
    int n_tiles;
    const float* part_val;
    const int32_t* part_idx;
    const float* part_z;
    const float* part_s;
    const float* cand_logit;
    const int32_t* node_tokens;
    float inv_t, epsilon, delta;
    int32_t* node_argmax;        // [B, n_nodes], required
    float* node_max;             // [B, n_nodes] scratch
    float* node_z;               // [B, n_nodes] scratch
    float* node_tau;             // [B, n_nodes], required
    float* node_prob;            // may be null
    int32_t* accept_len;
    int32_t* accept_nodes;
    int32_t* accept_tokens;
};
hipError_t typical_accept_launch(const DevicePlan& plan, int B, const TypicalAccept& a,
                                 hipStream_t stream);

// ------------------------------------------------------------------ attention
struct AttnShape {
    int B, N, Hq, Hkv, d, Lcap;
    int G;          // Hq / Hkv
    int rows;       // N * G query rows per (sequence, kv head)
    int waves;      // waves per workgroup
    int tile_r;     // bf16: 32-row query tiles per wave (1 or 2); fp32: 0 (16 rows per wave)
    int n_qblocks;  // query-row blocks per (sequence, kv head)
    int chunk;      // fp32: prefix keys per split (multiple of 64); bf16: fewest keys per chunk
    int n_splits;   // fp32: prefix splits
    int tree_merged;  // 1 (bf16): the tree keys join a sequence's last chunk when they fit
    int n_slots;    // fp32: partials per (sequence, kv head, query row); bf16: workgroups
                    // per (kv head, query-row block), shared out over the sequences'
                    // keys by the kernel
};
AttnShape attn_shape(medusa_dtype dt, int B, int N, int Hq, int Hkv, int d, int Lcap);
size_t attn_workspace_bytes(const AttnShape& s);
hipError_t attention_launch(medusa_dtype dt, const AttnShape& s, const DevicePlan& plan, float scale,
                            const void* q, const void* k_tree, const void* v_tree,
                            const void* k_cache, const void* v_cache, const int32_t* prefix_lens,
                            void* out, void* ws, hipStream_t stream);

// ------------------------------------------------------------------ verify + accept
// Body of medusa_verify_accept with the scratch area passed in (the caller's workspace, or
// the static scratch of medusa_verify_accept_noalloc).
medusa_status verify_accept_impl(const medusa_tree_plan* plan, medusa_dtype dt, int B, int H,
                                 int V, const void* node_hidden, const void* w_lm,
                                 const int32_t* node_tokens, int32_t* node_argmax,
                                 int32_t* accept_len, int32_t* accept_nodes,
                                 int32_t* accept_tokens, float* logits, void* ws,
                                 size_t ws_bytes, void* stream);

// ------------------------------------------------------------------ profiling
void prof_begin(const char* name, hipStream_t stream);
void prof_end(hipStream_t stream);

}  // namespace medusa
