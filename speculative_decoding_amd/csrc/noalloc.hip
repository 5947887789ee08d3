// medusa_verify_accept_noalloc: greedy verification and acceptance for callers that cannot
// allocate device memory (code under graph capture, tight serving loops, harnesses that
// forbid allocation).  It runs exactly the kernels of medusa_verify_accept; their scratch
// (per-tile argmax partials and the node argmax when the caller wants none) lives in the
// file-scope device array below instead of a caller workspace.
//
// The array's name is only a host-side stand-in in host code: its device address is taken
// once per device with hipGetSymbolAddress (with that device current) and kept; the kernels
// receive that address.  Every call on one device shares the array, so calls that overlap
// on one device (different streams, or threads) race on it.  Nothing in it needs to start
// at zero: the kernels write every partial before any is read.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"
#include "plan_impl.hpp"

namespace {

constexpr size_t kScratchBytes = MEDUSA_NOALLOC_SCRATCH_BYTES;   // per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch`, looked up on first use.
medusa_status scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return medusa_internal_hip_error(e);
    if (dev < 0 || dev >= kMaxDevices) return MEDUSA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return medusa_internal_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return MEDUSA_OK;
}

}  // namespace

extern "C" {

medusa_status medusa_verify_accept_noalloc(const medusa_tree_plan* plan, medusa_dtype dt, int B,
                                           int H, int V, const void* node_hidden,
                                           const void* w_lm, const int32_t* node_tokens,
                                           int32_t* node_argmax, int32_t* accept_len,
                                           int32_t* accept_nodes, int32_t* accept_tokens,
                                           float* logits, void* stream) {
    if (!plan || !node_hidden || !w_lm || !node_tokens || !accept_len || !accept_nodes ||
        !accept_tokens)
        return MEDUSA_ERR_NULL;
    const size_t need = medusa_verify_workspace(plan, dt, B, H, V);
    if (need == 0) return MEDUSA_ERR_SHAPE;
    if (need > kScratchBytes) return MEDUSA_ERR_WORKSPACE;
    medusa_status st = medusa_internal_device_check();
    if (st != MEDUSA_OK) return st;
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != MEDUSA_OK) return st;
    return medusa::verify_accept_impl(plan, dt, B, H, V, node_hidden, w_lm, node_tokens,
                                      node_argmax, accept_len, accept_nodes, accept_tokens,
                                      logits, ws, kScratchBytes, stream);
}

}  // extern "C"
