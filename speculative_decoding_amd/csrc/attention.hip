// Tree-masked attention (glossary "Medusa Heads", section "Attention arborescente et
// acceptation"; codewithpapers abstract): every tree node attends to the cached prefix and
// to the tree rows of its ancestors and itself, all nodes in one pass.
//
// Work split.  For one sequence b and one kv head g the query rows are the N*G
// (node, query head) pairs of that group; they share every key, so they are the M side of
// two MFMA contractions (scores and the value sum).  A workgroup takes 64 or 128 query rows
// (16 per wave) and one key range: a chunk of the prefix, or the tree keys.  Each 64-key
// block is staged in LDS (K row-major, V transposed) and shared by the waves.  Scores
// are computed transposed, S^T = K Q^T, so each lane owns one query row; its softmax
// state stays in registers and the value sum O^T = V^T P^T takes P^T straight from the
// score registers (the two 16-key score tiles give each lane the eight key slots of one
// 32-deep MFMA step; V^T is read from LDS with the same key order).  For bf16 the
// probabilities enter that MFMA as a hi + lo pair of bf16 values, so rounding them costs
// no more than fp32 accumulation would.  Partial (max, sum,
// unnormalised output) per key range go to the workspace; a second kernel combines them.
// The ancestor mask is one 64-bit word per (node, 64 keys).
#include "common.hpp"
#include "internal.hpp"

#include <type_traits>

namespace medusa {

namespace {

constexpr int kThreads = 256;     // the combine kernel
// Waves (16 query rows each) per attention workgroup: the K/V blocks staged in LDS are
// shared by all of them, so more waves mean fewer passes of the same keys through each CU.
// Measured: 8 waves help at 512 and more query rows per kv head (dense 256-node tree 105 ->
// 102 us, batched 70B 316 -> 300 us) and cost 3 us at 256 (the 8B tree: 22.5 -> 25.5 us),
// so attn_shape() takes 8 from 512 rows and 4 below.
constexpr int kAttnWavesSmall = 4;
constexpr int kAttnWavesLarge = 8;
constexpr int kAttnLargeRows = 512;
constexpr int kKeys = 64;          // keys staged per LDS block
// V^T row pitch: 64 keys + 12.  A 16-lane group of the value-operand reads (8 bytes per
// lane, rows l % 16) then covers 16 distinct bank pairs of the 32 banks; with + 8 rows l
// and l + 8 share banks.  Measured: batched 70B 279 -> 267 us, dense 96.6 -> 92.4 us
// (+ 4: 268 / 93.1).
constexpr int kVtPad = 12;

// Butterfly steps over lanes l ^ 16 and l ^ 32 on gfx950's lane-swap instructions (VALU,
// no trip through the LDS crossbar as a shuffle would take).  permlane16_swap(v, v) leaves
// rows 0, 0, 2, 2 of v (rows of 16 lanes) in its first result and rows 1, 1, 3, 3 in its
// second; permlane32_swap(v, v) leaves the low half twice and the high half twice.  Every
// lane of a pair combines the same two values in the same order.
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
    AttnShape s;
    DevicePlan plan;
    float scale_log2;
    const void* q;
    const void* k_tree;
    const void* v_tree;
    const void* k_cache;
    const void* v_cache;
    const int32_t* prefix_lens;
    void* out;
    float* ws_o;    // [B][Hkv][slots][rows][d]
    float* ws_ml;   // [B][Hkv][slots][rows][2]
};

template <typename T> struct Vt4;
template <> struct Vt4<bf16_t> {
    __device__ static __forceinline__ void load2(Frag<bf16_t>& f, const bf16_t* p0, const bf16_t* p1) {
        const uint2 a = *reinterpret_cast<const uint2*>(p0);
        const uint2 b = *reinterpret_cast<const uint2*>(p1);
        f.v = u32x4{a.x, a.y, b.x, b.y};
    }
    // p ~= hi + lo with hi = bf16(p) and lo = bf16(p - hi): the value sum runs as two
    // bf16 MFMAs, so the probabilities keep about 16 significant bits instead of 8.
    __device__ static __forceinline__ void pack(Frag<bf16_t>& hi, Frag<bf16_t>& lo, const float* p) {
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wh[i] = pack_bf16x2(p[2 * i], p[2 * i + 1]);
            wl[i] = pack_bf16x2(p[2 * i] - __uint_as_float(wh[i] << 16),
                                p[2 * i + 1] - __uint_as_float(wh[i] & 0xFFFF0000u));
        }
        hi.v = u32x4{wh[0], wh[1], wh[2], wh[3]};
        lo.v = u32x4{wl[0], wl[1], wl[2], wl[3]};
    }
    static constexpr bool kSplit = true;
    __device__ static __forceinline__ bf16_t elem(const u32x4& v, int e) {
        const uint32_t w = v[e >> 1];
        return (bf16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
    }
};
template <> struct Vt4<float> {
    __device__ static __forceinline__ void load2(Frag<float>& f, const float* p0, const float* p1) {
        f.lo = *reinterpret_cast<const u32x4*>(p0);
        f.hi = *reinterpret_cast<const u32x4*>(p1);
    }
    __device__ static __forceinline__ void pack(Frag<float>& f, Frag<float>& unused, const float* p) {
        f.lo = u32x4{__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]), __float_as_uint(p[3])};
        f.hi = u32x4{__float_as_uint(p[4]), __float_as_uint(p[5]), __float_as_uint(p[6]), __float_as_uint(p[7])};
        unused.zero();
    }
    static constexpr bool kSplit = false;
    __device__ static __forceinline__ float elem(const u32x4& v, int e) { return __uint_as_float(v[e]); }
};

template <typename T, int D, int NWV>
__global__ __launch_bounds__(NWV * 64) void attn_partial_kernel(const AttnArgs a) {
    constexpr int kAttnThreads = NWV * 64;
    constexpr int kAttnRows = 16 * NWV;
    constexpr int EPV = 16 / sizeof(T);
    constexpr int KP = D + 8;          // K row pitch (elements)
    constexpr int VP = kKeys + kVtPad;  // V^T row pitch
    constexpr int DS = D / 32;         // 32-deep steps over the head dim
    constexpr int DT = D / 16;         // 16-wide output tiles over the head dim
    __shared__ __align__(16) T Ks[kKeys * KP];
    __shared__ __align__(16) T Vt[D * VP];

    const AttnShape& sh = a.s;
    const int n_slots = sh.n_splits + 1;
    const int nblocks = sh.B * sh.Hkv * n_slots * sh.n_qblocks;
    int bid = xcd_logical_block(blockIdx.x, nblocks);
    const int qb = bid % sh.n_qblocks;
    bid /= sh.n_qblocks;
    const int slot = bid % n_slots;
    bid /= n_slots;
    const int g = bid % sh.Hkv;
    const int b = bid / sh.Hkv;

    const int L = min(max(a.prefix_lens[b], 0), sh.Lcap);
    const bool tree = slot == sh.n_splits;
    const int k_begin = tree ? 0 : slot * sh.chunk;
    const int k_end = tree ? sh.N : min(L, k_begin + sh.chunk);
    if (k_begin >= k_end) return;      // empty prefix chunk: the combine skips this slot

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int r = qb * kAttnRows + wave * 16 + ln;   // this lane's query row
    const bool row_ok = r < sh.rows;
    const int node = row_ok ? r / sh.G : 0;
    const int head = g * sh.G + (row_ok ? r % sh.G : 0);

    const T* q = static_cast<const T*>(a.q) + (((long long)b * sh.N + node) * sh.Hq + head) * D;
    Frag<T> qf[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
        if (row_ok) qf[ds].load(q + ds * 32 + 8 * lg);
        else qf[ds].zero();
    }

    const T* ksrc;
    const T* vsrc;
    long long kstride;   // elements between consecutive keys
    if (tree) {
        ksrc = static_cast<const T*>(a.k_tree) + ((long long)b * sh.N * sh.Hkv + g) * D;
        vsrc = static_cast<const T*>(a.v_tree) + ((long long)b * sh.N * sh.Hkv + g) * D;
    } else {
        ksrc = static_cast<const T*>(a.k_cache) + ((long long)b * sh.Lcap * sh.Hkv + g) * D;
        vsrc = static_cast<const T*>(a.v_cache) + ((long long)b * sh.Lcap * sh.Hkv + g) * D;
    }
    kstride = (long long)sh.Hkv * D;

    floatx4 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // K/V blocks are fetched into registers one block ahead, so the global loads of block
    // j+1 are in flight while block j is multiplied out of LDS.
    constexpr int VPR = D / EPV;                 // 16-byte vectors per key row
    constexpr int NV = kKeys * VPR / kAttnThreads;   // vectors per thread per block
    static_assert(NV * kAttnThreads == kKeys * VPR, "K/V block split over the threads");
    // K: consecutive threads read consecutive 16-byte pieces of a key row (coalesced, and
    // stored row-major).  V: consecutive threads take consecutive keys of one 16-byte column
    // piece, so the transposed scalar LDS stores of a wave hit 64 consecutive keys of one
    // V^T row (no bank conflicts) instead of 16 rows that all map to the same bank.
    // For bf16 a thread takes V in pairs of consecutive keys (vectors 2i and 2i+1: keys
    // 2q and 2q+1 of one column piece), so each V^T store is one 32-bit word holding both
    // keys: a wave's store covers 32 words of each of two V^T rows 32 banks apart, where
    // 16-bit stores put two lanes on every bank.
    constexpr bool kPairV = sizeof(T) == 2 && NV % 2 == 0;
    int kkey[NV], koff[NV], vkey[NV], voff[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int idx = threadIdx.x + j * kAttnThreads;
        kkey[j] = idx / VPR;
        koff[j] = kkey[j] * (int)kstride + (idx - kkey[j] * VPR) * EPV;
        if (kPairV) {
            const int u = threadIdx.x + (j >> 1) * kAttnThreads;     // (pair, piece) unit
            vkey[j] = 2 * (u % (kKeys / 2)) + (j & 1);
            voff[j] = vkey[j] * (int)kstride + (u / (kKeys / 2)) * EPV;
        } else {
            vkey[j] = idx % kKeys;
            voff[j] = vkey[j] * (int)kstride + (idx / kKeys) * EPV;
        }
    }
    u32x4 kr[NV], vr[NV];
    auto fetch = [&](int kb0) {
        const T* kb = ksrc + (long long)kb0 * kstride;
        const T* vb = vsrc + (long long)kb0 * kstride;
        if (kb0 + kKeys <= k_end) {          // a whole block: no per-key checks
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                kr[j] = *reinterpret_cast<const u32x4*>(kb + koff[j]);
                vr[j] = *reinterpret_cast<const u32x4*>(vb + voff[j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                kr[j] = u32x4{0u, 0u, 0u, 0u};
                vr[j] = kr[j];
                if (kb0 + kkey[j] < k_end) kr[j] = *reinterpret_cast<const u32x4*>(kb + koff[j]);
                if (kb0 + vkey[j] < k_end) vr[j] = *reinterpret_cast<const u32x4*>(vb + voff[j]);
            }
        }
    };

    // One 64-key block: TREE adds the ancestor mask; `whole` blocks of the prefix need no
    // per-key test at all (rows past the end have zero queries, so their scores stay
    // finite, and they are never stored).
    auto block = [&](auto tree_tag, int kb0) {
        constexpr bool TREE = decltype(tree_tag)::value;
        const bool whole = kb0 + kKeys <= k_end;
        const uint64_t mword = TREE && row_ok ? a.plan.mask[(long long)node * a.plan.mask_words + (kb0 >> 6)] : 0ull;
#pragma unroll
        for (int kb = 0; kb < kKeys; kb += 32) {
            if (kb0 + kb >= k_end) break;
            floatx4 sc[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                sc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < DS; ++ds) {
                    Frag<T> kf;
                    kf.load(Ks + (kb + t * 16 + ln) * KP + ds * 32 + 8 * lg);
                    mma(sc[t], kf, qf[ds]);
                }
            }
            // sc[t][j]: score of this lane's row against key kb0 + kb + 16 t + 4 lg + j
            float p[8];
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kl = kb + t * 16 + 4 * lg + j;        // key within the block
                    float v = sc[t][j] * a.scale_log2;
                    if (TREE) {
                        const bool ok = kb0 + kl < k_end && ((mword >> kl) & 1ull);
                        v = ok ? v : -INFINITY;
                    } else if (!whole) {
                        v = kb0 + kl < k_end ? v : -INFINITY;
                    }
                    p[t * 4 + j] = v;
                    mx = fmaxf(mx, v);
                }
            mx = max_xor32(max_xor16(mx));
            const float m_new = fmaxf(m_run, mx);
            // a row with every key of the step masked (only in the tree) keeps p = 0
            const float m_use = (TREE && m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = __builtin_amdgcn_exp2f(p[e] - m_use);
                psum += p[e];
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            Frag<T> pf, pf_lo;
            Vt4<T>::pack(pf, pf_lo, p);
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                o[t] *= alpha;
                Frag<T> vf;
                const T* vrow = Vt + (t * 16 + ln) * VP + kb + 4 * lg;
                Vt4<T>::load2(vf, vrow, vrow + 16);
                mma(o[t], vf, pf);
                if (Vt4<T>::kSplit) mma(o[t], vf, pf_lo);
            }
        }
    };

    fetch(k_begin);
    for (int kb0 = k_begin; kb0 < k_end; kb0 += kKeys) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            *reinterpret_cast<u32x4*>(Ks + kkey[j] * KP + (koff[j] - kkey[j] * (int)kstride)) = kr[j];
            const int vc8 = voff[j] - vkey[j] * (int)kstride;      // column piece * EPV
            if (kPairV) {
                if (j & 1) continue;
                // elements e of keys vkey[j] (even) and vkey[j] + 1: one V^T word
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    const uint32_t lo = vr[j][e >> 1], hi = vr[j + 1][e >> 1];
                    const uint32_t w = (e & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u))
                                               : ((lo & 0xFFFFu) | (hi << 16));
                    *reinterpret_cast<uint32_t*>(Vt + (vc8 + e) * VP + vkey[j]) = w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPV; ++e) Vt[(vc8 + e) * VP + vkey[j]] = Vt4<T>::elem(vr[j], e);
            }
        }
        __syncthreads();
        if (kb0 + kKeys < k_end) fetch(kb0 + kKeys);
        if (tree) block(std::true_type{}, kb0);
        else block(std::false_type{}, kb0);
    }
    l_run = sum_xor32(sum_xor16(l_run));
    if (!row_ok) return;
    const long long base = ((((long long)b * sh.Hkv + g) * n_slots + slot) * sh.rows + r);
    float* wo = a.ws_o + base * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
        *reinterpret_cast<floatx4*>(wo + t * 16 + 4 * lg) = o[t];
    if (lg == 0) {
        a.ws_ml[base * 2 + 0] = m_run;
        a.ws_ml[base * 2 + 1] = l_run;
    }
}

// One wave per (sequence, node, query head): combine the key ranges.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(const AttnArgs a) {
    using E = Elem<T>;
    constexpr int PER = D / kWave;
    const AttnShape& sh = a.s;
    const int row_id = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row_id >= sh.B * sh.N * sh.Hq) return;
    const int j = row_id % sh.Hq;
    const int i = (row_id / sh.Hq) % sh.N;
    const int b = row_id / (sh.Hq * sh.N);
    const int g = j / sh.G;
    const int r = i * sh.G + (j - g * sh.G);
    const int n_slots = sh.n_splits + 1;
    const int L = min(max(a.prefix_lens[b], 0), sh.Lcap);

    // every lane fetches one slot's (max, sum) so the slots are read in parallel
    const long long base0 = (((long long)b * sh.Hkv + g) * n_slots) * sh.rows + r;
    float den = 0.f;
    float num[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] = 0.f;
    float mx = -INFINITY;
    for (int s0 = 0; s0 < n_slots; s0 += kWave) {
        const int s = s0 + lane;
        const bool live = s < n_slots && (s == sh.n_splits || s * sh.chunk < L);
        const float ms = live ? a.ws_ml[(base0 + (long long)s * sh.rows) * 2] : -INFINITY;
        float m = ms;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) m = fmaxf(m, shfl_xor_f(m, o));
        mx = fmaxf(mx, m);
    }
    for (int s0 = 0; s0 < n_slots; s0 += kWave) {
        const int s = s0 + lane;
        const bool live = s < n_slots && (s == sh.n_splits || s * sh.chunk < L);
        const long long bs = base0 + (long long)s * sh.rows;
        const float w = live ? exp2f(a.ws_ml[bs * 2] - mx) : 0.f;
        float part = live ? w * a.ws_ml[bs * 2 + 1] : 0.f;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) part += shfl_xor_f(part, o);
        den += part;
        const int cnt = min(kWave, n_slots - s0);
        for (int j0 = 0; j0 < cnt; j0 += 8) {
            float ov[8][PER];
            float wj[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                wj[j] = __shfl(w, (j0 + j) & (kWave - 1), kWave);
                const bool use = j0 + j < cnt && wj[j] != 0.f;
                const long long bj = base0 + (long long)(s0 + j0 + j) * sh.rows;
#pragma unroll
                for (int e = 0; e < PER; ++e) ov[j][e] = use ? a.ws_o[bj * D + lane + kWave * e] : 0.f;
                if (!use) wj[j] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < PER; ++e) num[e] += wj[j] * ov[j][e];
        }
    }
    const float inv = 1.f / den;
    T* out = static_cast<T*>(a.out) + (((long long)b * sh.N + i) * sh.Hq + j) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[lane + kWave * e] = E::from_f32(num[e] * inv);
}

template <typename T, int D>
hipError_t launch_td(const AttnArgs& a, hipStream_t stream) {
    const AttnShape& s = a.s;
    const int nblocks = s.B * s.Hkv * (s.n_splits + 1) * s.n_qblocks;
    prof_begin("attn_partial", stream);
    if (s.waves == kAttnWavesLarge)
        hipLaunchKernelGGL((attn_partial_kernel<T, D, kAttnWavesLarge>), dim3(nblocks),
                           dim3(kAttnWavesLarge * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((attn_partial_kernel<T, D, kAttnWavesSmall>), dim3(nblocks),
                           dim3(kAttnWavesSmall * 64), 0, stream, a);
    prof_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int rows = s.B * s.N * s.Hq;
    prof_begin("attn_combine", stream);
    hipLaunchKernelGGL((attn_combine_kernel<T, D>), dim3((rows + 3) / 4), dim3(kThreads), 0, stream, a);
    prof_end(stream);
    return hipGetLastError();
}

}  // namespace

AttnShape attn_shape(int B, int N, int Hq, int Hkv, int d, int Lcap) {
    AttnShape s{};
    s.B = B; s.N = N; s.Hq = Hq; s.Hkv = Hkv; s.d = d; s.Lcap = Lcap;
    s.G = Hq / Hkv;
    s.rows = N * s.G;
    s.waves = s.rows >= kAttnLargeRows ? kAttnWavesLarge : kAttnWavesSmall;
    s.n_qblocks = (s.rows + 16 * s.waves - 1) / (16 * s.waves);
    // Split the prefix so that (a) the partial outputs (rows * d fp32 per split) stay
    // below about half the K/V bytes they summarise and (b) the grid still covers the
    // chip when there are few (sequence, kv head, query block) triples.
    const int max_splits = Lcap > 0 ? (Lcap + kKeys - 1) / kKeys : 1;
    int splits = Lcap / (2 * s.rows);
    const int base = B * Hkv * s.n_qblocks;
    // about 1024 waves in flight: with 2048 (twice the splits) the 8B tree took 22.6 + 8.9
    // us, against 22.2 + 7.8 here (7B shape 15.7 + 8.9 against 13.2 + 8.1)
    const int fill_blocks = 1024 / s.waves;
    const int fill = (fill_blocks + base - 1) / base;
    if (splits < fill) splits = fill;
    if (splits < 1) splits = 1;
    if (splits > max_splits) splits = max_splits;
    int chunk = Lcap > 0 ? (Lcap + splits - 1) / splits : kKeys;
    chunk = (chunk + kKeys - 1) / kKeys * kKeys;
    s.chunk = chunk;
    s.n_splits = Lcap > 0 ? (Lcap + chunk - 1) / chunk : 0;
    return s;
}

size_t attn_workspace_bytes(const AttnShape& s) {
    const size_t slots = (size_t)s.n_splits + 1;
    const size_t rows = (size_t)s.B * s.Hkv * slots * s.rows;
    return rows * (size_t)s.d * sizeof(float) + rows * 2 * sizeof(float) + 256;
}

hipError_t attention_launch(medusa_dtype dt, const AttnShape& s, const DevicePlan& plan, float scale,
                            const void* q, const void* k_tree, const void* v_tree,
                            const void* k_cache, const void* v_cache, const int32_t* prefix_lens,
                            void* out, void* ws, hipStream_t stream) {
    AttnArgs a;
    a.s = s;
    a.plan = plan;
    a.scale_log2 = scale * kLog2e;
    a.q = q; a.k_tree = k_tree; a.v_tree = v_tree; a.k_cache = k_cache; a.v_cache = v_cache;
    a.prefix_lens = prefix_lens;
    a.out = out;
    const size_t slots = (size_t)s.n_splits + 1;
    const size_t rows = (size_t)s.B * s.Hkv * slots * s.rows;
    a.ws_o = static_cast<float*>(ws);
    a.ws_ml = a.ws_o + rows * s.d;
    if (dt == MEDUSA_BF16) {
        return s.d == 64 ? launch_td<bf16_t, 64>(a, stream) : launch_td<bf16_t, 128>(a, stream);
    }
    return s.d == 64 ? launch_td<float, 64>(a, stream) : launch_td<float, 128>(a, stream);
}

}  // namespace medusa
