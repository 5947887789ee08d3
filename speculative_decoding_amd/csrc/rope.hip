// Rotary position embedding of the verifier's q and k, in place.
//
// The pages say nothing of positions.  A tree node continues the prefix at L + depth
// (siblings share a position: each branch is one possible continuation), and a real
// decoder layer rotates q and k by position.  This is that rotary form with element i
// paired with element i + d/2 of each head: for i < d/2, theta_i = base^(-2i/d),
// angle = pos*theta_i,
//     y_i = x_i cos - x_{i+d/2} sin,    y_{i+d/2} = x_{i+d/2} cos + x_i sin.
// The angle is formed and reduced modulo 2*pi in fp64 (positions reach 2^20, where an fp32
// angle would keep no fraction), then sin/cos and the rotation run in fp32 and the result
// is rounded to the storage type once.
#include "common.hpp"
#include "rope.hpp"

namespace medusa {

namespace {

constexpr int kRopeThreads = 256;

template <typename T> struct Quad;
template <> struct Quad<bf16_t> {
    static __device__ __forceinline__ void load(const bf16_t* p, float (&v)[4]) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        v[0] = __uint_as_float(w.x << 16);
        v[1] = __uint_as_float(w.x & 0xFFFF0000u);
        v[2] = __uint_as_float(w.y << 16);
        v[3] = __uint_as_float(w.y & 0xFFFF0000u);
    }
    static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[4]) {
        *reinterpret_cast<uint2*>(p) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
};
template <> struct Quad<float> {
    static __device__ __forceinline__ void load(const float* p, float (&v)[4]) {
        const float4 w = *reinterpret_cast<const float4*>(p);
        v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
    }
    static __device__ __forceinline__ void store(float* p, const float (&v)[4]) {
        *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]};
    }
};

// One thread per (row, head, four consecutive pairs); q heads first, then k heads.
template <typename T>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(const RopeArgs a) {
    const int quads = a.d / 8;                 // four-pair groups per head
    const int heads = a.Hq + a.Hkv;
    const long long idx = (long long)blockIdx.x * kRopeThreads + threadIdx.x;
    if (idx >= (long long)a.M * heads * quads) return;
    const int j = (int)(idx % quads);
    const long long t = idx / quads;
    const int h = (int)(t % heads);
    const long long m = t / heads;
    T* row = h < a.Hq ? static_cast<T*>(a.q) + (m * a.Hq + h) * a.d
                      : static_cast<T*>(a.k) + (m * a.Hkv + (h - a.Hq)) * a.d;
    T* lo_p = row + 4 * j;
    T* hi_p = row + a.d / 2 + 4 * j;
    float lo[4], hi[4];
    Quad<T>::load(lo_p, lo);
    Quad<T>::load(hi_p, hi);
    const double pos = (double)a.positions[m];
    constexpr double kTwoPi = 6.283185307179586476925286766559;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 4 * j + e;
        const double theta = exp2(-(2.0 * i / a.d) * a.log2_base);
        const double ang = pos * theta;
        const float r = (float)(ang - kTwoPi * rint(ang / kTwoPi));
        float s, c;
        sincosf(r, &s, &c);
        const float x0 = lo[e], x1 = hi[e];
        lo[e] = x0 * c - x1 * s;
        hi[e] = x1 * c + x0 * s;
    }
    Quad<T>::store(lo_p, lo);
    Quad<T>::store(hi_p, hi);
}

}  // namespace

hipError_t rope_launch(medusa_dtype dt, const RopeArgs& a, hipStream_t stream) {
    const long long total = (long long)a.M * (a.Hq + a.Hkv) * (a.d / 8);
    const dim3 grid((unsigned)((total + kRopeThreads - 1) / kRopeThreads));
    if (dt == MEDUSA_BF16)
        hipLaunchKernelGGL(rope_kernel<bf16_t>, grid, dim3(kRopeThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(kRopeThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace medusa
