// HBM read-bandwidth probe (probe.hip): declarations shared with the C API.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace medusa {

// Bytes one probe launch reads from a buffer of `bytes` (whole 8 KiB blocks).
long long hbm_probe_bytes(size_t bytes);
hipError_t hbm_probe_launch(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
// out[0] = shader clock ticks, out[1] = 100 MHz ticks over one MFMA-bound workgroup's run.
hipError_t clock_probe_launch(unsigned long long* out, uint32_t* sink, int cus, hipStream_t stream);

}  // namespace medusa
