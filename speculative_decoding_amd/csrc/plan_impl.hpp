// Internal layout of the opaque medusa_tree_plan and host helpers shared by the C-ABI files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <vector>

#include "../../include/medusa.h"
#include "internal.hpp"

struct medusa_tree_plan {
    int n_nodes = 0;
    int max_depth = 0;
    int mask_words = 0;
    std::vector<int32_t> parent, depth, rank;
    std::vector<uint64_t> mask;
    // device image: parent | depth | rank | mask
    size_t off_depth = 0, off_rank = 0, off_mask = 0, image_bytes = 0;
    std::vector<unsigned char> image;
    unsigned char* dev = nullptr;   // caller-owned buffer holding the image, once uploaded
};

// MEDUSA_OK if a HIP device is visible, else MEDUSA_ERR_NO_DEVICE.
medusa_status medusa_internal_device_check();
// Records `e` as this thread's last HIP error and returns MEDUSA_ERR_HIP.
medusa_status medusa_internal_hip_error(hipError_t e);

inline medusa::DevicePlan medusa_internal_device_plan(const medusa_tree_plan* p) {
    medusa::DevicePlan d;
    d.parent = reinterpret_cast<const int32_t*>(p->dev);
    d.depth = reinterpret_cast<const int32_t*>(p->dev + p->off_depth);
    d.rank = reinterpret_cast<const int32_t*>(p->dev + p->off_rank);
    d.mask = reinterpret_cast<const uint64_t*>(p->dev + p->off_mask);
    d.n_nodes = p->n_nodes;
    d.max_depth = p->max_depth;
    d.mask_words = p->mask_words;
    return d;
}
