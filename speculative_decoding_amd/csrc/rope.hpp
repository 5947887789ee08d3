// Rotary positions of the verifier (rope.hip): declarations shared with the C API.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/medusa.h"

namespace medusa {

struct RopeArgs {
    void* q;                    // [M, Hq, d], rotated in place
    void* k;                    // [M, Hkv, d], rotated in place
    const int32_t* positions;   // [M]
    double log2_base;           // log2 of the rotary base
    int M, Hq, Hkv, d;
};
hipError_t rope_launch(medusa_dtype dt, const RopeArgs& args, hipStream_t stream);

}  // namespace medusa
