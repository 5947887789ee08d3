// Next round of the decode loop (tree.hip): declarations shared with the C API.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace medusa {

// Next round: accepted branch rows into the KV cache, next h and root (byte sizes of one
// K/V row, Hkv*d elements, and of one hidden row are multiples of 16).
struct AdvanceArgs {
    const int32_t* accept_len;
    const int32_t* accept_nodes;    // [B, max_depth + 1]
    const int32_t* accept_tokens;
    const void* k_tree;             // [B, n_nodes, row_bytes]
    const void* v_tree;
    const void* node_hidden;        // [B, n_nodes, hidden_bytes]
    void* k_cache;                  // [B, Lcap, row_bytes]
    void* v_cache;
    int32_t* prefix_lens;
    void* hidden_out;               // [B, hidden_bytes]
    int32_t* root_out;
    int32_t* overflow;              // may be null
    int n_nodes, max_depth, Lcap;
    int row_bytes, hidden_bytes;
};
hipError_t advance_launch(const AdvanceArgs& args, int B, hipStream_t stream);

}  // namespace medusa
