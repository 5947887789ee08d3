/*
 * medusa.h — C ABI of libmedusa: one Medusa decode step on MI355X (gfx950).
 *
 * The method (from the web pages on Medusa):
 *   - heads      Ultralytics glossary "Medusa Heads", section "Comment les têtes
 *                prédisent les tokens suivants": head k reads the last hidden state h,
 *                applies one feed-forward layer with SiLU and a residual connection,
 *                then a projection to the vocabulary: logits_k = W2_k (h + SiLU(W1_k h + b1_k)).
 *                lm_head scores position t+1, head k scores t+k+1.
 *   - tree       same page, section "Attention arborescente et acceptation": the top
 *                candidates of the heads combine as a Cartesian product into a tree of
 *                continuations sharing prefixes; a sparse tree of the most accurate
 *                combinations (64 nodes) beats a dense one (256 nodes).
 *   - attention  same section: every candidate is appended to the input at once and a
 *                mask lets each token see only its ancestors in the tree (this library:
 *                its ancestors and itself), on top of the cached prefix.
 *   - verify     same section: under greedy decoding a candidate is accepted when it
 *                equals the model's first choice; the longest accepted branch is kept.
 *                The deepest accepted node's own first choice is emitted after it
 *                (blog "Medusa no contexto de LLMs", section "o que significa medusa na
 *                prática de deploy": a rejected candidate falls back to the
 *                conventionally generated token).
 *
 * Conventions (every call):
 *   - Tensors are device pointers to contiguous, row-major arrays, 16-byte aligned.
 *     Weights are [out, in] (the nn.Linear layout of the glossary page's example).
 *     Floating tensors are MEDUSA_BF16 (bf16 storage, fp32 accumulation) or
 *     MEDUSA_F32; logits and top-k values are always fp32; ids are int32.
 *   - The caller owns every buffer, including the workspace, whose size the
 *     *_workspace query returns.  No call allocates device memory; the tree plan is
 *     the only library-owned object (host memory) and is uploaded into a
 *     caller-provided device buffer.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue;
 *     nothing synchronises.  Outputs are valid once the stream has synchronised.
 *   - Errors the host can detect (null pointers, bad shapes, unsupported sizes,
 *     malformed trees, small workspace, no device) return a status before anything
 *     is enqueued and leave outputs untouched.  Nothing prints, aborts or throws.
 *     Token ids read from device memory are not validated on the host: an id outside
 *     [0, V) gathers a zero row instead of reading out of bounds.
 *   - Plans are immutable after creation and may be shared between threads; calls on
 *     different streams may run concurrently when their outputs and workspaces differ.
 */
#ifndef MEDUSA_H
#define MEDUSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MEDUSA_OK = 0,
    MEDUSA_ERR_NULL = 1,          /* a required pointer is NULL                         */
    MEDUSA_ERR_SHAPE = 2,         /* a size is out of range or inconsistent             */
    MEDUSA_ERR_UNSUPPORTED = 3,   /* dtype / head dim / top-k size not supported        */
    MEDUSA_ERR_TREE = 4,          /* malformed tree: not prefix-closed, duplicate, ...  */
    MEDUSA_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than the query's answer  */
    MEDUSA_ERR_NO_DEVICE = 6,     /* no HIP device visible                              */
    MEDUSA_ERR_HIP = 7,           /* a HIP runtime call failed (see medusa_last_hip_error) */
    MEDUSA_ERR_PLAN_NOT_ON_DEVICE = 8  /* the plan was not uploaded (medusa_tree_plan_upload) */
} medusa_status;

typedef enum { MEDUSA_F32 = 0, MEDUSA_BF16 = 1 } medusa_dtype;

#define MEDUSA_MAX_TOPK 64       /* largest top-k per head                                 */
#define MEDUSA_MAX_HEADS 8       /* largest number of Medusa heads                         */
#define MEDUSA_MAX_NODES 1024    /* largest tree, root included                            */

/* ------------------------------------------------------------------ tree plans
 * A node is a rank tuple (i_1, ..., i_d): at depth d it carries head d's rank-i_d
 * candidate, under the node (i_1, ..., i_{d-1}); node 0 is the root (the base model's own
 * next token).  Nodes are stored breadth first: depth ascending, then tuple
 * lexicographically ascending.  Bit j of mask row i is set iff node j is an ancestor of
 * node i or j == i.  (Glossary "Medusa Heads", section "Attention arborescente et
 * acceptation".)  All plan functions are host-only and never touch a device, except
 * medusa_tree_plan_upload. */
typedef struct medusa_tree_plan medusa_tree_plan;

/* paths: host [n_paths, max_depth] int32 rank tuples, each padded with -1 after its last
 * rank; the root is implicit and must not be listed.  Rejects (MEDUSA_ERR_TREE) duplicate
 * tuples, negative ranks inside a tuple, ranks >= MEDUSA_MAX_TOPK, and sets that are not
 * closed under taking prefixes.  n_paths + 1 <= MEDUSA_MAX_NODES. */
medusa_status medusa_tree_plan_create(const int32_t* paths, int n_paths, int max_depth,
                                      medusa_tree_plan** out);

/* The dense tree: the full Cartesian product of tree_s[0..depth) at every depth. */
medusa_status medusa_tree_plan_full(const int32_t* tree_s, int depth, medusa_tree_plan** out);

/* The sparse tree of n_nodes nodes (root included) built from the most accurate
 * combinations: every rank tuple t of the Cartesian product of tree_s (depths 1..depth)
 * is scored prod_d acc[(d-1)*acc_stride + t_d] (double, multiplied in depth order); the
 * n_nodes-1 best by (score descending, depth ascending, tuple ascending) are kept.
 * acc: host doubles, per-head rank accuracies, each row descending in (0, 1). */
medusa_status medusa_tree_plan_from_accuracy(const double* acc, int acc_stride,
                                             const int32_t* tree_s, int depth, int n_nodes,
                                             medusa_tree_plan** out);

/* Expected accepted length of a plan under per-head rank accuracies (same section: the
 * sparse tree is the set of most accurate combinations, and a 64-node such tree is said to
 * beat a 256-node dense one).  acc[(d-1)*acc_stride + r] is the probability that head d's
 * rank-r candidate is the base model's next token at depth d (host doubles in [0, 1],
 * heads independent, acc_rows >= the plan's max_depth, acc_stride >= every rank used + 1).
 * Siblings exclude one another, so E[a] = sum over non-root nodes of the product of acc
 * along the node's path; *out receives it (0 for a root-only plan).  Host only. */
medusa_status medusa_tree_plan_expected_accept(const medusa_tree_plan* plan, const double* acc,
                                               int acc_stride, int acc_rows, double* out);

/* Shape of a plan: node count, deepest depth, 64-bit words per mask row. */
medusa_status medusa_tree_plan_info(const medusa_tree_plan* plan, int* n_nodes, int* max_depth,
                                    int* mask_words);

/* Host copies of the plan arrays ([N] each, mask [N, mask_words]); any may be NULL. */
medusa_status medusa_tree_plan_arrays(const medusa_tree_plan* plan, int32_t* parent,
                                      int32_t* depth, int32_t* rank, uint64_t* mask);

/* Bytes of device memory the plan needs, and its upload: copies the plan's arrays into
 * `device_buf` (caller-owned, >= medusa_tree_plan_device_bytes bytes, 256-B aligned)
 * on `stream` and records the buffer in the plan.  The buffer must stay allocated while
 * the plan is used on the device.  Uploading again replaces the recorded buffer. */
size_t medusa_tree_plan_device_bytes(const medusa_tree_plan* plan);
medusa_status medusa_tree_plan_upload(medusa_tree_plan* plan, void* device_buf, size_t bytes,
                                      void* stream);
void medusa_tree_plan_destroy(medusa_tree_plan* plan);

/* ------------------------------------------------------------------ 1. heads
 * For every sequence b and head k (glossary "Medusa Heads", section "Comment les têtes
 * prédisent les tokens suivants"):
 *     z = W1_k h_b + b1_k;   u_bk = rnd(h_b + SiLU(z));   logits_bk = W2_k u_bk
 * with SiLU(x) = x / (1 + e^-x) and rnd() rounding to the dtype (bf16: nearest even).
 * Then the top-s_k ids of logits_bk, ordered by value descending, ties to the lower id
 * (section "Attention arborescente et acceptation": the best hypotheses of each head).
 * If w_lm is given the bootstrap root r_b = argmax(W_lm h_b) (lowest id on ties) is also
 * computed, through the same projection code path as the heads.
 *
 *   hidden   [B, H]        w1 [K, H, H]   b1 [K, H]   w2 [K, V, H]   w_lm [V, H] or NULL
 *   s        HOST [K]      top-k per head, 1..MEDUSA_MAX_TOPK, each <= V; s_max = max(s)
 *   topk_ids [B, K, s_max] int32, entries past s_k are -1
 *   topk_vals[B, K, s_max] fp32, entries past s_k are 0
 *   root_ids [B] int32 or NULL (written iff w_lm != NULL)
 *   u_out    [B, K, H] dtype or NULL (head hidden states; kept in the workspace if NULL)
 *   logits   [B, K+1, V] fp32 or NULL (slot K holds lm_head(h) iff w_lm != NULL)
 * Limits: 1 <= B <= 64, 1 <= K <= MEDUSA_MAX_HEADS, H % 32 == 0, 32 <= H <= 16384,
 * 1 <= V <= 262144 (the top-s candidates of at most 2048 vocabulary tiles of 128 rows are
 * merged per head; a larger V returns MEDUSA_ERR_SHAPE). */
medusa_status medusa_heads_forward(medusa_dtype dt, int B, int H, int V, int K,
                                   const void* hidden, const void* w1, const void* b1,
                                   const void* w2, const void* w_lm, const int32_t* s,
                                   int s_max, int32_t* topk_ids, float* topk_vals,
                                   int32_t* root_ids, void* u_out, float* logits, void* ws,
                                   size_t ws_bytes, void* stream);
size_t medusa_heads_workspace(medusa_dtype dt, int B, int H, int V, int K, int s_max);

/* ------------------------------------------------------------------ 2. tree
 * Fill the tree's tokens (glossary, "Attention arborescente et acceptation": head 2
 * proposes the same tokens under every head-1 branch):
 *     node_tokens[b, 0] = root_ids[b]
 *     node_tokens[b, i] = topk_ids[b, depth(i)-1, rank(i)]       (i >= 1)
 *     position_ids[b, i] = prefix_lens[b] + depth(i)             (siblings share a position)
 *   s HOST [K]: every plan rank at depth d must be < s[d-1]; plan depth <= K.
 *   prefix_lens [B] int32 device or NULL (then positions start at 0); position_ids may be NULL. */
medusa_status medusa_build_tree(const medusa_tree_plan* plan, int B, int K, int s_max,
                                const int32_t* s, const int32_t* root_ids,
                                const int32_t* topk_ids, const int32_t* prefix_lens,
                                int32_t* node_tokens, int32_t* position_ids, void* stream);

/* ------------------------------------------------------------------ 3. tree attention
 * For node i and query head j (kv head g = j / (Hq/Hkv), contiguous groups):
 *     keys   = k_cache[b, 0..L_b, g]  followed by  k_tree[b, m, g] for m in anc(i) U {i}
 *     o[b,i,j] = rnd( softmax(scale * q[b,i,j] . keys) . values )
 * (glossary, "Attention arborescente et acceptation": each candidate sees only its tree
 * ancestors; codewithpapers abstract: tree-based attention verifies all candidates in one
 * step).  scale <= 0 selects 1/sqrt(d).
 *   q [B,N,Hq,d]  k_tree, v_tree [B,N,Hkv,d]  k_cache, v_cache [B,Lcap,Hkv,d]
 *   prefix_lens [B] int32 device, each in [0, Lcap] (larger values are clamped to Lcap)
 *   out [B,N,Hq,d] dtype.   d in {64, 128}; Hq % Hkv == 0; Lcap <= 2^20. */
medusa_status medusa_tree_attention(const medusa_tree_plan* plan, medusa_dtype dt, int B, int Hq,
                                    int Hkv, int d, int Lcap, float scale, const void* q,
                                    const void* k_tree, const void* v_tree, const void* k_cache,
                                    const void* v_cache, const int32_t* prefix_lens, void* out,
                                    void* ws, size_t ws_bytes, void* stream);
size_t medusa_attention_workspace(const medusa_tree_plan* plan, medusa_dtype dt, int B, int Hq,
                                  int Hkv, int d, int Lcap);

/* ------------------------------------------------------------------ 4. verify + accept
 * logits_i = W_lm node_hidden_i; a_i = argmax (lowest id on ties).  accepted(0) holds;
 * node i >= 1 is accepted iff its parent is accepted and node_tokens[i] == a_parent(i).
 * accept_len = deepest accepted depth a; accept_nodes = the node path root..i* (-1
 * padded to D+1); accept_tokens = the candidates on that path (depths 1..a) followed by
 * a_{i*} (-1 padded to D+1).  (Glossary, "Attention arborescente et acceptation".)
 *   node_hidden [B,N,H] dtype   w_lm [V,H]   node_tokens [B,N] int32
 *   node_argmax [B,N] or NULL   accept_len [B]   accept_nodes, accept_tokens [B, D+1]
 *   logits [B,N,V] fp32 or NULL.  H % 32 == 0. */
medusa_status medusa_verify_accept(const medusa_tree_plan* plan, medusa_dtype dt, int B, int H,
                                   int V, const void* node_hidden, const void* w_lm,
                                   const int32_t* node_tokens, int32_t* node_argmax,
                                   int32_t* accept_len, int32_t* accept_nodes,
                                   int32_t* accept_tokens, float* logits, void* ws,
                                   size_t ws_bytes, void* stream);
size_t medusa_verify_workspace(const medusa_tree_plan* plan, medusa_dtype dt, int B, int H, int V);

/* medusa_verify_accept without a workspace, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, kernels and results as medusa_verify_accept, minus ws/ws_bytes: the scratch
 * (per-tile argmax partials; the node argmax when node_argmax is NULL) is a static device
 * array of MEDUSA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  The call allocates nothing.  Problems whose medusa_verify_workspace()
 * exceeds that size return MEDUSA_ERR_WORKSPACE before anything is enqueued.  All calls on
 * one GPU share its array: calls that overlap on one GPU (other streams or threads) race,
 * so a caller serialises them. */
#define MEDUSA_NOALLOC_SCRATCH_BYTES 4194304   /* 4 MiB */
medusa_status medusa_verify_accept_noalloc(const medusa_tree_plan* plan, medusa_dtype dt, int B,
                                           int H, int V, const void* node_hidden,
                                           const void* w_lm, const int32_t* node_tokens,
                                           int32_t* node_argmax, int32_t* accept_len,
                                           int32_t* accept_nodes, int32_t* accept_tokens,
                                           float* logits, void* stream);

/* Typical acceptance, for sampling (same section: every candidate whose probability under
 * the base model exceeds a threshold tied to the entropy of that distribution is kept; more
 * tokens pass, exact agreement with the base model's distribution is given up).  The page
 * gives no formula; this library reads it as
 *     p_i = softmax(logits_i / temperature) over the vocabulary,  H_i = -sum p_i ln p_i,
 *     tau_i = min(epsilon, delta * exp(-H_i)),
 *     node c >= 1 accepted iff its parent i is accepted and p_i(node_tokens[c]) > tau_i.
 * Several siblings may pass; the kept branch ends at the deepest accepted node, the lowest
 * index among equals, and emits its candidates and then that node's argmax a_{i*}, as in
 * medusa_verify_accept (same output layouts).  Optional outputs: node_argmax [B,N] int32,
 * node_prob [B,N] fp32 (p of each node's token under its parent's distribution; 1 for the
 * root), node_tau [B,N] fp32 (tau_i), logits [B,N,V] fp32.  Arithmetic is fp32; the
 * softmax sums are merged over vocabulary tiles in a fixed order.
 * 1e-6 <= temperature <= 1e6; epsilon, delta finite and >= 0 (else MEDUSA_ERR_SHAPE).
 * ws/ws_bytes: at least medusa_verify_typical_workspace() bytes. */
medusa_status medusa_verify_accept_typical(const medusa_tree_plan* plan, medusa_dtype dt, int B,
                                           int H, int V, const void* node_hidden, const void* w_lm,
                                           const int32_t* node_tokens, float temperature,
                                           float epsilon, float delta, int32_t* node_argmax,
                                           float* node_prob, float* node_tau, int32_t* accept_len,
                                           int32_t* accept_nodes, int32_t* accept_tokens,
                                           float* logits, void* ws, size_t ws_bytes,
                                           void* stream);
size_t medusa_verify_typical_workspace(const medusa_tree_plan* plan, medusa_dtype dt, int B,
                                       int H, int V);

/* ------------------------------------------------------------------ 5. next round
 * Commit each sequence's accepted branch and set up the next step (glossary, "Attention
 * arborescente et acceptation": the longest accepted branch is kept and its last hidden
 * state feeds the heads in the next round).  With a = accept_len[b], the branch
 * accept_nodes[b, 0..a] (root first) and L = prefix_lens[b]:
 *     k_cache[b, L + j] = k_tree[b, accept_nodes[b, j]],  v likewise,   j = 0..a
 *     prefix_lens[b] = L + a + 1
 *     hidden_out[b] = node_hidden[b, accept_nodes[b, a]]   (the next step's h)
 *     root_out[b]   = accept_tokens[b, a]                  (the next step's root: the bonus)
 * These are exactly the cache rows and the state plain greedy decoding reaches after the
 * emitted tokens.  A branch that does not fit (L + a + 1 > Lcap) changes nothing for its
 * sequence and sets overflow[b] = 1 (0 otherwise) when overflow is not NULL.
 *   accept_len [B], accept_nodes, accept_tokens [B, D+1] int32 (as written by
 *   medusa_verify_accept; D = the plan's depth)   k_tree, v_tree [B,N,Hkv,d] dtype
 *   node_hidden [B,N,H] dtype   k_cache, v_cache [B,Lcap,Hkv,d] and prefix_lens [B] int32,
 *   updated in place   hidden_out [B,H] dtype (typically the h buffer the next
 *   medusa_heads_forward reads; must not overlap node_hidden)   root_out [B] int32
 *   overflow [B] int32 or NULL.   (Hkv*d) % 8 == 0 and H % 8 == 0; 16-byte aligned rows. */
medusa_status medusa_advance(const medusa_tree_plan* plan, medusa_dtype dt, int B, int H, int Hkv,
                             int d, int Lcap, const int32_t* accept_len,
                             const int32_t* accept_nodes, const int32_t* accept_tokens,
                             const void* k_tree, const void* v_tree, const void* node_hidden,
                             void* k_cache, void* v_cache, int32_t* prefix_lens, void* hidden_out,
                             int32_t* root_out, int32_t* overflow, void* stream);

/* ------------------------------------------------------------------ measurement
 * HBM read-bandwidth probe (not part of the method): streams the first
 * medusa_hbm_probe_bytes(bytes) bytes of `buf` (whole 8 KiB blocks) once, with the access
 * pattern of the heads' GEMV (64 lanes x 16 contiguous bytes per load, non-temporal), and
 * writes `sink` (a device uint32) only in the rare case its checksum equals one fixed
 * value.  Timing it with events on `stream` gives the read ceiling that the streaming
 * kernels are compared with.  buf 16-byte aligned and at least 8 KiB. */
size_t medusa_hbm_probe_bytes(size_t bytes);
medusa_status medusa_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);
/* Clock probe (not part of the method): four workgroups per CU run a chain of bf16 MFMAs
 * on every SIMD; one wave reads the shader clock counter and the constant 100 MHz counter
 * before and after its share and writes the two tick counts to ticks[0..1] (device
 * uint64).  ticks[0] / ticks[1] * 100 MHz is the shader clock under MFMA load.  `sink` (a
 * device uint32) is written only in an impossible case; it keeps the MFMAs live. */
medusa_status medusa_clock_probe(uint64_t* ticks, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------ one-layer verifier
 * A stand-in for the frozen base model that scores the tree (not part of the method):
 * embedding gather, Q/K/V projections, and the attention output projection with the
 * residual.  M = B*N rows.
 *   proxy_qkv:  x_m = embed[tokens[m]]; q = rnd(Wq x) [M, Hq*d]; k = rnd(Wk x),
 *               v = rnd(Wv x) [M, Hkv*d].  Wq [Hq*d, H], Wk/Wv [Hkv*d, H].
 *   proxy_out:  node_hidden_m = rnd(embed[tokens[m]] + Wo o_m)  [M, H]; Wo [H, Hq*d],
 *               o [M, Hq*d].   H % 32 == 0 and (Hq*d) % 32 == 0.
 * ws/ws_bytes: scratch for contraction-slice partial sums, at least
 * medusa_proxy_workspace() bytes (the same buffer serves both calls). */
size_t medusa_proxy_workspace(medusa_dtype dt, int M, int H, int Hq, int Hkv, int d);
medusa_status medusa_proxy_qkv(medusa_dtype dt, int M, int H, int V, int Hq, int Hkv, int d,
                               const int32_t* tokens, const void* embed, const void* wq,
                               const void* wk, const void* wv, void* q, void* k, void* v,
                               void* ws, size_t ws_bytes, void* stream);
/* Rotary positions for the verifier's q and k, in place (not on the pages; a real decoder
 * layer needs it): with element i of a head paired with element i + d/2, for i < d/2,
 *     theta_i = base^(-2i/d),  a = positions[m] * theta_i,
 *     (x_i, x_{i+d/2}) <- (x_i cos a - x_{i+d/2} sin a,  x_{i+d/2} cos a + x_i sin a),
 * then rounded to dt once.  Tree nodes take positions[m] = L + depth (position_ids of
 * medusa_build_tree).  The angle is reduced in fp64, the rotation is fp32.
 *   q [M, Hq, d] and k [M, Hkv, d] dtype, updated   positions [M] int32.
 *   d % 8 == 0, 1 < base (finite). */
medusa_status medusa_rope(medusa_dtype dt, int M, int Hq, int Hkv, int d, const int32_t* positions,
                          float base, void* q, void* k, void* stream);

medusa_status medusa_proxy_out(medusa_dtype dt, int M, int H, int V, int Hq, int d,
                               const int32_t* tokens, const void* embed, const void* o,
                               const void* wo, void* node_hidden, void* ws, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------------ misc */
const char* medusa_status_string(medusa_status status);
/* hipError_t of the last MEDUSA_ERR_HIP returned on this thread (0 if none). */
int medusa_last_hip_error(void);
int medusa_version(void);

/* Per-kernel timing for measurement runs: while enabled, every kernel this library
 * launches is bracketed by two HIP events on its stream.  medusa_profile_query waits
 * for those events and returns the summed GPU time and launch count of every launch of
 * `kernel` since the last reset (kernel names: "heads_ffn", "heads_vocab", "heads_merge",
 * "build_tree", "proxy_qkv", "attn_partial", "attn_combine", "proxy_out",
 * "verify_lmhead", "verify_accept").  Not thread-safe; at most 8192 launches are
 * recorded between resets (later ones are not timed). */
medusa_status medusa_profile_enable(int on);
/* Restrict timing to the launches of one kernel (NULL: time every kernel).  Each timed
 * launch adds two event records to its stream, which costs a few microseconds. */
medusa_status medusa_profile_only(const char* kernel);
medusa_status medusa_profile_reset(void);
medusa_status medusa_profile_query(const char* kernel, double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif
#endif /* MEDUSA_H */
