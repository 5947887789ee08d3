// Tree-masked attention (glossary "Medusa Heads", section "Attention arborescente et
// acceptation"; codewithpapers abstract): every tree node attends to the cached prefix and
// to the tree rows of its ancestors and itself, all nodes in one pass.
//
// Work split.  For one sequence b and one kv head g the query rows are the N*G
// (node, query head) pairs of that group; they share every key, so they are the M side of
// two MFMA contractions (scores and the value sum).  A workgroup takes a block of query
// rows and one key range: a chunk of the prefix, possibly with the tree keys.  Partial
// (max, sum, unnormalised output) per key range go to the workspace; a second kernel
// combines them.  The ancestor mask is one 64-bit word per (node, 64 keys).
//
// bf16 (attn_tile_kernel): the workgroups of a (kv head, query-row block) share out the
// keys of all sequences by their actual prefix lengths (attn_find_slot), so ragged batches
// fill one round of the chip instead of reserving slots for the longest possible prefix.
// 32 x 32 x 16 MFMA tiles, one 32-row query tile per wave, four or eight waves sharing the
// K/V blocks staged in LDS.  Scores
// are computed transposed, S^T = K Q^T: a lane owns one query column of each 32-row tile
// (shared with the lane 32 apart) and 16 keys of every 32.  The value sum O^T = V^T P^T
// takes P^T straight from the score registers as fp16 and V^T from LDS as fp16: bf16 values
// convert to fp16 exactly from 2^-14 up to 65504, so the probabilities keep 11 significant
// bits where bf16 keeps 8, in one MFMA instead of a hi + lo pair.  A workgroup whose
// accumulators come out non-finite (a value beyond fp16's range, or inf/NaN inputs)
// computes its rows again in fp32 on the vector units.
// The running maximum is kept lazily: the accumulators are rescaled only when a row's
// maximum grows by more than 2^8, so probabilities stay below 256 and fp16 holds them.
//
// fp32 (attn_partial_kernel): 16 x 16 x 4 fp32 MFMAs, 16 query rows per wave.
#include "common.hpp"
#include "internal.hpp"

#include <type_traits>

namespace medusa {

namespace {

constexpr int kThreads = 256;     // the combine kernel
// fp32 kernel: waves (16 query rows each) per workgroup: the K/V blocks staged in LDS are
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
    float* ws_o;    // fp32 kernel: [B][Hkv][slots][rows][d] unnormalised partial outputs;
                    // bf16 kernel: [workgroup][rows][d] normalised partials in fp32, written
                    // only by the fp32 recomputation
    float* ws_ml;   // fp32 kernel: the same rows x (running maximum, sum);
                    // bf16 kernel: [workgroup][rows] x (maximum, sum, 1 if the row is in
                    // ws_o else 0, unused)
    uint16_t* ws_h; // bf16 kernel: [workgroup][rows][d] normalised partial outputs as fp16
    int* ws_plan;   // bf16: [B] first workgroup slot of each sequence, then [B] slot counts
};

// ---- the bf16 kernel's split of the keys ----
// The workgroups of one (kv head, query-row block) unit, sh.n_slots of them, share out the
// keys of all sequences: sequence b takes n_b consecutive slots, ceil(L_b / C) prefix
// chunks of C keys and the tree keys, which join the last chunk when they fit into its
// spare room and take a slot of their own otherwise (an empty prefix: one slot, the tree).
// C is the smallest multiple of 64, at least sh.chunk, for which the slots of all
// sequences fit the unit's workgroups; the longest slot bounds the kernel's time.
__device__ __forceinline__ int attn_slots_of(int L, int N, int C) {
    const int np = (L + C - 1) / C;
    return np == 0 ? 1 : np + (L + N > np * C ? 1 : 0);
}
// Whole-wave sum / maximum on DPP row steps and four lane reads; every lane gets it.
__device__ __forceinline__ int wave_sum_int(int v) {
    v += dpp_i<kDppXor1>(v);
    v += dpp_i<kDppXor2>(v);
    v += dpp_i<kDppHalfMirror>(v);
    v += dpp_i<kDppMirror>(v);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
__device__ __forceinline__ int wave_max_int(int v) {
    v = max(v, dpp_i<kDppXor1>(v));
    v = max(v, dpp_i<kDppXor2>(v));
    v = max(v, dpp_i<kDppHalfMirror>(v));
    v = max(v, dpp_i<kDppMirror>(v));
    return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_scan_int(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const int u = __shfl_up(v, m, 64);
        if (lane >= m) v += u;
    }
    return v;
}
// Hardware block h runs on XCD h % 8 as that XCD's (h / 8)-th block.  Group j = (slot,
// kv head), slot-major, goes to XCD j % 8 with its nq row blocks in consecutive places
// there, so they share one L2 for the keys they read; the groups start in order, so the
// low slots, which hold work whenever the sequences need them, go first to distinct CUs.
__device__ __forceinline__ void attn_block_map(int h, int groups, int nq, int& grp, int& qb) {
    const int full = groups & ~7;              // groups in whole rounds of the 8 XCDs
    if (h < full * nq) {
        const int x = h & 7, k = h >> 3;
        grp = (k / nq) * 8 + x;
        qb = k % nq;
    } else {
        const int t = h - full * nq;
        grp = full + t / nq;
        qb = t % nq;
    }
}
struct AttnSlot {
    int b;            // sequence; -1: an idle workgroup
    int n;            // the sequence's slot count
    int p_begin, p_end;
    bool with_tree;
};
// Called by every lane of a wave; the result is the same in all lanes.  `plan_out`, when
// not null, receives every sequence's first slot and slot count.
__device__ AttnSlot attn_find_slot(const int32_t* lens, int B, int Lcap, int N, int S, int cmin,
                                   int slot, int* plan_out) {
    const int lane = threadIdx.x & 63;
    // lane l holds sequence b0 + l; up to 64 sequences the lengths stay in registers
    const int L0 = lane < B ? min(max(lens[lane], 0), Lcap) : 0;
    auto len_of = [&](int b0) {
        if (B <= 64) return L0;
        return b0 + lane < B ? min(max(lens[b0 + lane], 0), Lcap) : 0;
    };
    auto total_slots = [&](int C) {
        int t = 0;
        for (int b0 = 0; b0 < B; b0 += 64) t += wave_sum_int(b0 + lane < B ? attn_slots_of(len_of(b0), N, C) : 0);
        return t;
    };
    int sumw = 0, maxw = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int w = b0 + lane < B ? len_of(b0) + N : 0;
        sumw += wave_sum_int(w);
        maxw = max(maxw, wave_max_int(w));
    }
    // C >= sum(W) / S is necessary (a sequence of W keys needs W / C slots or more), and
    // with one sequence sufficient; `hi` (one slot per sequence, B <= S) always fits.
    int lo = max(max(1, cmin / 64), (sumw + 64 * S - 1) / (64 * S));
    int hi = max(lo, (maxw + 63) / 64);
    if (total_slots(64 * lo) <= S) {
        hi = lo;
    } else {
        ++lo;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (total_slots(64 * mid) <= S) hi = mid;
            else lo = mid + 1;
        }
    }
    const int C = 64 * hi;
    AttnSlot r{-1, 0, 0, 0, false};
    int carry = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int b = b0 + lane;
        const int L = len_of(b0);
        const int n = b < B ? attn_slots_of(L, N, C) : 0;
        const int off = carry + wave_scan_int(n) - n;
        if (plan_out && b < B) {
            plan_out[b] = off;
            plan_out[B + b] = n;
        }
        const unsigned long long hit = __ballot(b < B && off <= slot && slot < off + n);
        if (hit) {
            const int src = __ffsll((long long)hit) - 1;
            const int j = slot - __shfl(off, src, 64);
            const int nb = __shfl(n, src, 64);
            const int Lb = __shfl(L, src, 64);
            r.b = b0 + src;
            r.n = nb;
            r.p_begin = min(j * C, Lb);      // the tree's own slot: an empty prefix range
            r.p_end = min((j + 1) * C, Lb);
            r.with_tree = j == nb - 1;
        }
        carry = __shfl(off + n, 63, 64);        // off already counts the earlier chunks
    }
    return r;
}

template <typename T> struct Vt4;
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
    const int n_slots = sh.n_slots;
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

// ------------------------------------------------------------------ bf16: 32 x 32 tiles

// Element e (0..7) of eight bf16 values held as four words, as fp32 (exact).
__device__ __forceinline__ float bf16_elem(const u32x4& v, int e) {
    const uint32_t w = v[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// acc[32x32] += A[32 x 16] * B[16 x 32]: lane l supplies row (l % 32) of A and column
// (l % 32) of B at contraction slots 8*(l/32) .. 8*(l/32)+7 (any slot -> index map shared by
// A and B is allowed).  Lane l holds acc[8*(v/4) + 4*(l/32) + v%4][l % 32] in register v.
__device__ __forceinline__ void mma32_bf16(floatx16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32_f16(floatx16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}
// Two fp32 values as one word of fp16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    const f16x2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}
// Element e (0..7) of eight fp16 values held as four words, as fp32 (exact).
// acc + the two fp16 halves of w, in fp32 (one v_dot2_f32_f16 against (1, 1)): the row
// sums then add exactly the fp16 probabilities that the value MFMAs multiply.
__device__ __forceinline__ float sum_f16x2(uint32_t w, float acc) {
    const f16x2 one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
}
__device__ __forceinline__ float f16_elem(const u32x4& v, int e) {
    // through a scalar: a bit cast applied to the vector subscript itself reads word 0
    const uint32_t w = v[e >> 1];
    const f16x2 p = __builtin_bit_cast(f16x2, w);
    return static_cast<float>(p[e & 1]);
}
// The rows [row0, row0 + nrows) of one (sequence, kv head) over one key range, in fp32 on
// the vector units straight from global memory, one row per thread: scores, their maximum
// and sum, then the output divided by the sum, 32 head-dim elements at a time, into the
// fp32 rows at wo_base (and (maximum, sum, 1) into ml_base).  Written for correctness
// only: it serves the rare key range whose fp16 value path overflowed.  Kept out of line
// so that it adds no registers to the tiled kernel.
template <int D>
__device__ __noinline__ void attn_rows_fp32(const bf16_t* q, const bf16_t* kpre, const bf16_t* vpre,
                                            const bf16_t* ktr, const bf16_t* vtr,
                                            const uint64_t* mask, int mask_words, float* wo_base,
                                            float* ml_base, int rows, int N, int G, int Hq,
                                            int g, long long kstride, float scale_log2, int row0,
                                            int nrows, int p_begin, int p_end, bool with_tree) {
    const int r = row0 + (int)threadIdx.x;
    if ((int)threadIdx.x >= nrows || r >= rows) return;
    const int node = r / G;
    const int head = g * G + r % G;
    const bf16_t* qr = q + ((long long)node * Hq + head) * D;
    // keys j < n_pre are prefix rows p_begin + j; the next N (with_tree) are tree rows
    const int n_pre = p_end - p_begin;
    const int n_all = n_pre + (with_tree ? N : 0);
    auto row_k = [&](int j) { return j < n_pre ? kpre + (p_begin + j) * kstride : ktr + (j - n_pre) * kstride; };
    auto row_v = [&](int j) { return j < n_pre ? vpre + (p_begin + j) * kstride : vtr + (j - n_pre) * kstride; };
    auto visible = [&](int j) {
        if (j < n_pre) return true;
        const int m = j - n_pre;
        return ((mask[(long long)node * mask_words + (m >> 6)] >> (m & 63)) & 1ull) != 0;
    };
    auto score = [&](int j) {
        const bf16_t* kr = row_k(j);
        float s = 0.f;
        for (int e = 0; e < D; ++e) s += bf16_to_f32(qr[e]) * bf16_to_f32(kr[e]);
        return s * scale_log2;
    };
    float m = -INFINITY;
    for (int j = 0; j < n_all; ++j)
        if (visible(j)) m = fmaxf(m, score(j));
    const float mb = m == -INFINITY ? 0.f : m;
    float l = 0.f;
    for (int j = 0; j < n_all; ++j)
        if (visible(j)) l += exp2f(score(j) - mb);
    // stored normalised and in fp32: values beyond fp16's range, whose contributions the
    // merge may cancel, keep their full precision
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* wo = wo_base + (long long)r * D;
    for (int c = 0; c < D; c += 32) {
        float acc[32];
        for (int e = 0; e < 32; ++e) acc[e] = 0.f;
        for (int j = 0; j < n_all; ++j) {
            if (!visible(j)) continue;
            const float p = exp2f(score(j) - mb);
            const bf16_t* vr = row_v(j) + c;
            for (int e = 0; e < 32; ++e) acc[e] += p * bf16_to_f32(vr[e]);
        }
        for (int e = 0; e < 32; ++e) wo[c + e] = acc[e] * inv;
    }
    ml_base[4 * r + 0] = m;
    ml_base[4 * r + 1] = l;
    ml_base[4 * r + 2] = 1.f;
}

// Compile-time tuning overrides (0: chosen from the shape).
#ifndef MEDUSA_ATTN_WGS
#define MEDUSA_ATTN_WGS 0          // bf16: workgroups per launch (0: one round of the chip)
#endif
#ifndef MEDUSA_ATTN_MERGE_J
#define MEDUSA_ATTN_MERGE_J 4      // bf16 merge: slots whose loads are in flight together
#endif
#ifndef MEDUSA_ATTN_MIN_CHUNK
#define MEDUSA_ATTN_MIN_CHUNK 256  // bf16: fewest prefix keys per chunk
#endif
#ifndef MEDUSA_ATTN_PRIO
#define MEDUSA_ATTN_PRIO 0    // raise the wave priority around its MFMA runs
#endif


#ifndef MEDUSA_ATTN_W
#define MEDUSA_ATTN_W 0       // waves per workgroup (0: chosen from the shape)
#endif

constexpr int kTileKeys = 64;       // keys per LDS block
constexpr float kLazyMax = 8.f;     // rescale once a row maximum grows by more than 2^8

// D: head dim (64 or 128); NW: waves per workgroup (4 or 8), one 32-row query tile each.
// The NW waves share every K / V block staged in LDS, so eight waves halve the staging per
// query row; they need 256 query rows per kv head to fill their tiles.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_tile_kernel(const AttnArgs a) {
    constexpr int R = 1;                 // 32-row query tiles per wave
    constexpr int kTileThreads = NW * 64;
    constexpr int KB = kTileKeys;
    constexpr int KP = D + 8;            // K row pitch: rows 4 banks apart, 8 rows cover 32
    constexpr int VP = KB + 8;           // V^T row pitch: rows 4 banks apart, 8 rows cover 32
    constexpr int KS = D / 16;           // 16-deep steps over the head dim
    constexpr int DT = D / 32;           // 32-row tiles of O^T over the head dim
    constexpr int ROWS = 32 * R * NW;
    constexpr int KVEC = KB * D / 8;                 // 16-byte K pieces per block
    constexpr int KPT = KVEC / kTileThreads;         // ... per thread
    constexpr int VUNITS = (KB / 4) * (D / 8);       // V units: 4 keys x 8 head-dim elements
    static_assert(KPT * kTileThreads == KVEC, "K block split over the threads");
    static_assert(VUNITS <= kTileThreads, "one V unit per thread at most");
    __shared__ __align__(16) bf16_t Ks[2][KB * KP];
    __shared__ __align__(16) uint16_t Vt[2][D * VP];

    const AttnShape& sh = a.s;
    const int n_slots = sh.n_slots;
    int grp, qb;
    attn_block_map(blockIdx.x, n_slots * sh.Hkv, sh.n_qblocks, grp, qb);
    const int slot = grp / sh.Hkv;
    const int g = grp % sh.Hkv;
    const int bid = (g * n_slots + slot) * sh.n_qblocks + qb;     // this workgroup's partial block
    const AttnSlot as = attn_find_slot(a.prefix_lens, sh.B, sh.Lcap, sh.N, n_slots, sh.chunk, slot,
                                       bid == 0 && threadIdx.x < 64 ? a.ws_plan : nullptr);
    // uniform values: keep them (and every loop bound) in scalar registers
    const int b = __builtin_amdgcn_readfirstlane(as.b);
    if (b < 0) return;                 // more workgroups than slots
    const int n_seq_slots = __builtin_amdgcn_readfirstlane(as.n);
    const int p_begin = __builtin_amdgcn_readfirstlane(as.p_begin);
    const int p_end = __builtin_amdgcn_readfirstlane(as.p_end);
    const bool with_tree = __builtin_amdgcn_readfirstlane((int)as.with_tree) != 0;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // Q^T operands: lane l holds query row (tile base + l % 32) at head-dim slots
    // 16 ks + 8 (l / 32) .. + 7 of every 16-deep step.
    u32x4 qf[R][KS];
    int node[R];
    bool row_ok[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const int r = qb * ROWS + (wave * R + t) * 32 + l32;
        row_ok[t] = r < sh.rows;
        node[t] = row_ok[t] ? r / sh.G : 0;
        const int head = g * sh.G + (row_ok[t] ? r % sh.G : 0);
        const bf16_t* q = static_cast<const bf16_t*>(a.q) +
                          (((long long)b * sh.N + node[t]) * sh.Hq + head) * D + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[t][ks] = row_ok[t] ? *reinterpret_cast<const u32x4*>(q + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
    }

    const bf16_t* const kpre = static_cast<const bf16_t*>(a.k_cache) + ((long long)b * sh.Lcap * sh.Hkv + g) * D;
    const bf16_t* const vpre = static_cast<const bf16_t*>(a.v_cache) + ((long long)b * sh.Lcap * sh.Hkv + g) * D;
    const bf16_t* const ktr = static_cast<const bf16_t*>(a.k_tree) + ((long long)b * sh.N * sh.Hkv + g) * D;
    const bf16_t* const vtr = static_cast<const bf16_t*>(a.v_tree) + ((long long)b * sh.N * sh.Hkv + g) * D;
    const long long kstride = (long long)sh.Hkv * D;   // elements between consecutive keys
    // the key range the loop below walks: the prefix chunk, then the tree keys
    const bf16_t* ksrc = kpre;
    const bf16_t* vsrc = vpre;
    int k_begin = p_begin, k_end = p_end;

    // Staging.  K: consecutive threads take consecutive 16-byte pieces of a key row.  V: a
    // thread takes one unit of 4 consecutive keys x 8 head-dim elements (four 16-byte
    // loads) and writes each element's 4 keys as one 8-byte word of V^T; the 16 lanes that
    // share an element write 128 consecutive bytes.
    // Per-lane offsets (elements) within a block; the block's base pointer is uniform.
    int kkey[KPT], koff[KPT], kls[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int idx = tid + j * kTileThreads;
        kkey[j] = idx / (D / 8);
        koff[j] = kkey[j] * (int)kstride + (idx % (D / 8)) * 8;
        kls[j] = kkey[j] * KP + (idx % (D / 8)) * 8;
    }
    constexpr bool kAllV = VUNITS == kTileThreads;
    const bool vact = kAllV || tid < VUNITS;
    const int vq = tid % (KB / 4);      // key quad
    const int vp = tid / (KB / 4);      // head-dim piece of 8
    const int voff = 4 * vq * (int)kstride + vp * 8;
    // V^T keeps each 16-key group permuted (key 8a + 4b + c at 8b + 4a + c), so the eight
    // keys one lane feeds to a value MFMA are eight consecutive elements: one 16-byte read
    const int vls = (8 * vp) * VP + 4 * ((vq & ~3) | ((vq & 1) << 1) | ((vq >> 1) & 1));
    u32x4 kr[KPT], vr[4];
    auto fetch = [&](int kb0) {
        const bf16_t* kb = ksrc + (long long)kb0 * kstride;
        const bf16_t* vb = vsrc + (long long)kb0 * kstride;
        if (kb0 + KB <= k_end) {          // a whole block: no per-key tests
#pragma unroll
            for (int j = 0; j < KPT; ++j) kr[j] = *reinterpret_cast<const u32x4*>(kb + koff[j]);
            if (vact) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vr[i] = *reinterpret_cast<const u32x4*>(vb + voff + i * (int)kstride);
            }
        } else {
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                kr[j] = u32x4{0u, 0u, 0u, 0u};
                if (kb0 + kkey[j] < k_end) kr[j] = *reinterpret_cast<const u32x4*>(kb + koff[j]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vr[i] = u32x4{0u, 0u, 0u, 0u};
                if (vact && kb0 + 4 * vq + i < k_end)
                    vr[i] = *reinterpret_cast<const u32x4*>(vb + voff + i * (int)kstride);
            }
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) *reinterpret_cast<u32x4*>(&Ks[buf][kls[j]]) = kr[j];
        if (vact) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {      // fp16: exact in fp16's normal range
                uint2 w;
                w.x = pack_f16x2(bf16_elem(vr[0], e), bf16_elem(vr[1], e));
                w.y = pack_f16x2(bf16_elem(vr[2], e), bf16_elem(vr[3], e));
                *reinterpret_cast<uint2*>(&Vt[buf][vls + e * VP]) = w;
            }
        }
    };

    floatx16 o[R][DT];
    float m_used[R], l_sum[R];

    // One 64-key block out of LDS buffer `buf`, as two 32-key halves: scores, lazily
    // rescaled softmax, value sum.  Register v of score tile sc[t] is key
    // kb0 + 32 h + 8 (v/4) + 4 hi + v%4.  MASK: 0 a whole prefix block, 1 the prefix's last
    // block (keys past the end), 2 tree keys (the ancestor mask; it has no bit past the
    // last node, whose K/V rows stage as zeros).
    const float c2 = a.scale_log2;
    auto block = [&](int buf, int kb0, auto mask_tag) {
        constexpr int MASK = decltype(mask_tag)::value;
        uint64_t mw[R];
#pragma unroll
        for (int t = 0; t < R; ++t)
            mw[t] = (MASK == 2 && row_ok[t]) ? a.plan.mask[(long long)node[t] * a.plan.mask_words + (kb0 >> 6)] : 0ull;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (MASK != 0 && kb0 + 32 * h >= k_end) break;
            floatx16 sc[R];
#pragma unroll
            for (int t = 0; t < R; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) sc[t][v] = 0.f;
            if (MEDUSA_ATTN_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(&Ks[buf][(32 * h + l32) * KP + 16 * ks + 8 * hi]);
#pragma unroll
                for (int t = 0; t < R; ++t) mma32_bf16(sc[t], kf, qf[t][ks]);
            }
            if (MEDUSA_ATTN_PRIO) __builtin_amdgcn_s_setprio(0);
            // row maxima of the raw scores (the scale is positive), masked keys at -inf
            float mx[R];
#pragma unroll
            for (int t = 0; t < R; ++t) {
                if (MASK == 2) {
                    const uint32_t bits = (uint32_t)(mw[t] >> (32 * h + 4 * hi));
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (!((bits >> (8 * (v >> 2) + (v & 3))) & 1u)) sc[t][v] = -INFINITY;
                } else if (MASK == 1) {
                    const int left = k_end - (kb0 + 32 * h + 4 * hi);
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (8 * (v >> 2) + (v & 3) >= left) sc[t][v] = -INFINITY;
                }
                float m = sc[t][0];
#pragma unroll
                for (int v = 1; v < 16; ++v) m = fmaxf(m, sc[t][v]);
                mx[t] = max_xor32(m) * c2;
            }
            bool grow = false;
#pragma unroll
            for (int t = 0; t < R; ++t) grow |= mx[t] > m_used[t] + kLazyMax;
            if (__any(grow)) {
#pragma unroll
                for (int t = 0; t < R; ++t) {
                    const float m_new = fmaxf(m_used[t], mx[t]);
                    const float alpha = m_used[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_used[t] - m_new);
                    l_sum[t] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) o[t][dt] *= alpha;
                    m_used[t] = m_new;
                }
            }
            // probabilities p = 2^(s c - m) as the P^T operands: pf[t][kk] holds registers
            // 8 kk .. 8 kk + 7
            u32x4 pf[R][2];
#pragma unroll
            for (int t = 0; t < R; ++t) {
                const float mb = m_used[t] == -INFINITY ? 0.f : m_used[t];
                float ls = 0.f;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][8 * kk + 2 * w], c2, -mb));
                        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][8 * kk + 2 * w + 1], c2, -mb));
                        const uint32_t pw = pack_f16x2(p0, p1);
                        pf[t][kk][w] = pw;
                        ls = sum_f16x2(pw, ls);
                    }
                l_sum[t] += ls;
            }
            // value sum: V^T rows 32 dt + l % 32, the eight keys of this lane's P^T slots
            if (MEDUSA_ATTN_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const u32x4 vf = *reinterpret_cast<const u32x4*>(
                        &Vt[buf][(32 * dt + l32) * VP + 32 * h + 16 * kk + 8 * hi]);
#pragma unroll
                    for (int t = 0; t < R; ++t) mma32_f16(o[t][dt], vf, pf[t][kk]);
                }
            if (MEDUSA_ATTN_PRIO) __builtin_amdgcn_s_setprio(0);
        }
    };
    using NoMask = std::integral_constant<int, 0>;
    using BoundMask = std::integral_constant<int, 1>;
    using TreeMask = std::integral_constant<int, 2>;

    // The whole key range, double-buffered: block j+1 is written into the other LDS buffer
    // while block j is used, and the loads of block j+2 are issued right after; one barrier
    // per block.  Every block but the last is whole; the last, which may end inside the
    // block, runs after the loop.  The tree keys and a prefix chunk run separate copies of
    // the loop (with and without the ancestor mask).
    auto run = [&](auto tree_tag) {
        constexpr bool TREE = decltype(tree_tag)::value;
        fetch(k_begin);
        stage(0);
        if (k_begin + KB < k_end) fetch(k_begin + KB);
        __syncthreads();
        int buf = 0;
        int kb0 = k_begin;
        for (; kb0 + KB < k_end; kb0 += KB) {
            if (TREE) block(buf, kb0, TreeMask{});
            else block(buf, kb0, NoMask{});
            stage(buf ^ 1);
            if (kb0 + 2 * KB < k_end) fetch(kb0 + 2 * KB);
            __syncthreads();
            buf ^= 1;
        }
        if (TREE) block(buf, kb0, TreeMask{});
        else if (kb0 + KB == k_end) block(buf, kb0, NoMask{});
        else block(buf, kb0, BoundMask{});
        __syncthreads();       // the LDS buffers are free again
    };
#pragma unroll
    for (int t = 0; t < R; ++t) {
        m_used[t] = -INFINITY;
        l_sum[t] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[t][dt][v] = 0.f;
    }
    if (p_begin < p_end) run(std::false_type{});
    if (with_tree) {
        ksrc = ktr;
        vsrc = vtr;
        k_begin = 0;
        k_end = sh.N;
        run(std::true_type{});
    }

    // A value beyond fp16's range (or an inf/NaN input) leaves a non-finite accumulator:
    // the workgroup's rows are then computed again in fp32 on the vector units.
    bool bad = false;
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) bad |= !__builtin_isfinite(o[t][dt][v]);
    // this workgroup's partial rows: row r of the kv head at slot_base + r
    const long long slot_base = ((long long)bid - qb) * ROWS;
    bf16_t* const out = static_cast<bf16_t*>(a.out);
    const bool fallback = __syncthreads_or(bad);
    if (fallback)
        attn_rows_fp32<D>(static_cast<const bf16_t*>(a.q) + (long long)b * sh.N * sh.Hq * D, kpre,
                          vpre, ktr, vtr, a.plan.mask, a.plan.mask_words, a.ws_o + slot_base * D,
                          a.ws_ml + slot_base * 4, sh.rows, sh.N, sh.G, sh.Hq, g, kstride,
                          a.scale_log2, qb * ROWS, ROWS, p_begin, p_end, with_tree);

    // The only slot of its sequence writes the attention output straight from its
    // registers.
    const bool only = n_seq_slots == 1;
    if (only && !fallback) {
#pragma unroll
        for (int t = 0; t < R; ++t) {
            const float inv = 1.f / sum_xor32(l_sum[t]);
            if (!row_ok[t]) continue;
            const int r = qb * ROWS + (wave * R + t) * 32 + l32;
            bf16_t* orow = out + (((long long)b * sh.N + r / sh.G) * sh.Hq + g * sh.G + r % sh.G) * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * j + 4 * hi) =
                        uint2{pack_bf16x2(o[t][dt][4 * j] * inv, o[t][dt][4 * j + 1] * inv),
                              pack_bf16x2(o[t][dt][4 * j + 2] * inv, o[t][dt][4 * j + 3] * inv)};
        }
        return;
    }

    // After the fp32 recomputation, the only slot normalises the partial it wrote.
    if (only) {
        __syncthreads();
        for (int i = tid; i < ROWS * (D / 8); i += kTileThreads) {
            const int r = qb * ROWS + i / (D / 8);
            if (r >= sh.rows) continue;
            const int part = i % (D / 8);
            const long long bs = slot_base + r;
            const floatx4 f0 = *reinterpret_cast<const floatx4*>(a.ws_o + bs * D + part * 8);
            const floatx4 f1 = *reinterpret_cast<const floatx4*>(a.ws_o + bs * D + part * 8 + 4);
            const float v[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
            bf16_t* orow = out + (((long long)b * sh.N + r / sh.G) * sh.Hq + g * sh.G + r % sh.G) * D + part * 8;
            *reinterpret_cast<u32x4*>(orow) = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                    pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
        }
        return;
    }

    // Otherwise the partial goes to the workspace for attn_merge_kernel: the normalised
    // output o / l as fp16 (a convex combination of values that all fit fp16 on this
    // path), and the running maximum and sum.
    if (!fallback) {
#pragma unroll
        for (int t = 0; t < R; ++t) {
            const float l_row = sum_xor32(l_sum[t]);
            if (!row_ok[t]) continue;
            const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
            const int r = qb * ROWS + (wave * R + t) * 32 + l32;
            const long long base = slot_base + r;
            uint16_t* wo = a.ws_h + base * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<uint2*>(wo + 32 * dt + 8 * j + 4 * hi) =
                        uint2{pack_f16x2(o[t][dt][4 * j] * inv, o[t][dt][4 * j + 1] * inv),
                              pack_f16x2(o[t][dt][4 * j + 2] * inv, o[t][dt][4 * j + 3] * inv)};
            if (hi == 0)
                *reinterpret_cast<floatx4*>(a.ws_ml + base * 4) = floatx4{m_used[t], l_row, 0.f, 0.f};
        }
    }
}

// bf16: merge the partials of the sequences that took more than one slot (a sequence with
// one slot had its output written directly).  Sixteen threads per query row, eight
// head-dim elements each; MEDUSA_ATTN_MERGE_J slots' loads are issued before any is used.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnArgs a) {
    constexpr int TPR = D / 8;                       // threads per row
    constexpr int MAXJ = MEDUSA_ATTN_MERGE_J;        // slots per pass
    const AttnShape& sh = a.s;
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)sh.B * sh.Hkv * sh.rows * TPR;
    if (gid >= total) return;
    const int part = (int)(gid % TPR);
    const long long row_id = gid / TPR;              // (b, g, r)
    const int r = (int)(row_id % sh.rows);
    const int bg = (int)(row_id / sh.rows);
    const int b = bg / sh.Hkv;
    const int g = bg % sh.Hkv;
    const int n = a.ws_plan[sh.B + b];               // the sequence's slots
    if (n <= 1) return;                              // written directly by its only slot
    const int first = a.ws_plan[b];
    const int per = 32 * sh.waves;                   // query rows per workgroup
    const int qb = r / per;
    // slot j's partial row: workgroup ((g n_slots + first + j) n_qblocks + qb), row r % per
    const long long base0 = (((long long)g * sh.n_slots + first) * sh.n_qblocks + qb) * per + r % per;
    const long long step = (long long)sh.n_qblocks * per;
    // one pass with a running maximum
    float mx = -INFINITY, den = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n; s0 += MAXJ) {
        floatx4 ml[MAXJ];
        u32x4 hv[MAXJ];
#pragma unroll
        for (int u = 0; u < MAXJ; ++u) {
            const int sl = min(s0 + u, n - 1);
            const long long bs = base0 + (long long)sl * step;
            ml[u] = *reinterpret_cast<const floatx4*>(a.ws_ml + bs * 4);
            hv[u] = *reinterpret_cast<const u32x4*>(a.ws_h + bs * D + part * 8);
        }
#pragma unroll
        for (int u = 0; u < MAXJ; ++u) {
            if (s0 + u >= n || ml[u][0] == -INFINITY) continue;
            // slot u holds o_u / l_u (fp16, or fp32 after the recomputation) and its
            // maximum m_u and sum l_u
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = f16_elem(hv[u], e);
            if (ml[u][2] != 0.f) {
                const float* f = a.ws_o + (base0 + (long long)(s0 + u) * step) * D + part * 8;
                const floatx4 f0 = *reinterpret_cast<const floatx4*>(f);
                const floatx4 f1 = *reinterpret_cast<const floatx4*>(f + 4);
                v[0] = f0[0]; v[1] = f0[1]; v[2] = f0[2]; v[3] = f0[3];
                v[4] = f1[0]; v[5] = f1[1]; v[6] = f1[2]; v[7] = f1[3];
            }
            const float m_new = fmaxf(mx, ml[u][0]);
            const float alpha = mx == -INFINITY ? 0.f : exp2f(mx - m_new);
            const float w = exp2f(ml[u][0] - m_new) * ml[u][1];
            den = den * alpha + w;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = acc[e] * alpha + w * v[e];
            mx = m_new;
        }
    }
    const float inv = 1.f / den;
    bf16_t* orow = static_cast<bf16_t*>(a.out) +
                   (((long long)b * sh.N + r / sh.G) * sh.Hq + g * sh.G + r % sh.G) * D + part * 8;
    *reinterpret_cast<u32x4*>(orow) =
        u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
              pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
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
    const int n_slots = sh.n_slots;
    const int L = min(max(a.prefix_lens[b], 0), sh.Lcap);
    // live slots: prefix chunks that hold keys, and the tree keys (their own slot, or the
    // last live chunk's)
    const int last = L > 0 ? (L - 1) / sh.chunk : 0;
    auto is_live = [&](int s) {
        if (s >= n_slots) return false;
        if (sh.tree_merged) return s <= last;
        return s == sh.n_splits || s * sh.chunk < L;
    };

    // every lane fetches one slot's (max, sum) so the slots are read in parallel
    const long long base0 = (((long long)b * sh.Hkv + g) * n_slots) * sh.rows + r;
    float den = 0.f;
    float num[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] = 0.f;
    float mx = -INFINITY;
    for (int s0 = 0; s0 < n_slots; s0 += kWave) {
        const int s = s0 + lane;
        const bool live = is_live(s);
        const float ms = live ? a.ws_ml[(base0 + (long long)s * sh.rows) * 2] : -INFINITY;
        float m = ms;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) m = fmaxf(m, shfl_xor_f(m, o));
        mx = fmaxf(mx, m);
    }
    for (int s0 = 0; s0 < n_slots; s0 += kWave) {
        const int s = s0 + lane;
        const bool live = is_live(s);
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
    if constexpr (std::is_same<T, bf16_t>::value) {
        const int nblocks = s.Hkv * s.n_slots * s.n_qblocks;
        prof_begin("attn_partial", stream);
        if (s.waves == 8)
            hipLaunchKernelGGL((attn_tile_kernel<D, 8>), dim3(nblocks), dim3(8 * 64), 0, stream, a);
        else
            hipLaunchKernelGGL((attn_tile_kernel<D, 4>), dim3(nblocks), dim3(4 * 64), 0, stream, a);
        prof_end(stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const long long threads = (long long)s.B * s.Hkv * s.rows * (D / 8);
        prof_begin("attn_combine", stream);
        hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                           stream, a);
        prof_end(stream);
        return hipGetLastError();
    } else {
        const int nblocks = s.B * s.Hkv * s.n_slots * s.n_qblocks;
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
}

}  // namespace

AttnShape attn_shape(medusa_dtype dt, int B, int N, int Hq, int Hkv, int d, int Lcap) {
    AttnShape s{};
    s.B = B; s.N = N; s.Hq = Hq; s.Hkv = Hkv; s.d = d; s.Lcap = Lcap;
    s.G = Hq / Hkv;
    s.rows = N * s.G;
    if (dt == MEDUSA_BF16) {
        // One 32-row query tile per wave.  Eight waves from 512 query rows per kv head
        // (two or more blocks of 256 rows sharing every staged K/V block), four below.
        // Measured (tile kernel, us, 4 -> 8 waves): dense tree 70.8 -> 58.9, batched 70B
        // 152 -> 134, 8B shape (256 rows) 22.2 -> 26.5.
        s.tile_r = 1;
        s.waves = s.rows >= 512 ? 8 : 4;
#if MEDUSA_ATTN_W
        s.waves = MEDUSA_ATTN_W;
#endif
        const int per = 32 * s.waves;
        s.n_qblocks = (s.rows + per - 1) / per;
        // Workgroups per (kv head, row block) unit: as many as one round of the chip holds
        // (one 8-wave or two 4-wave workgroups per CU), at least one per sequence; the
        // kernel shares them out over the actual key counts (attn_find_slot).
        const int wgs = MEDUSA_ATTN_WGS > 0 ? MEDUSA_ATTN_WGS : (s.waves == 8 ? 256 : 512);
        const int units = Hkv * s.n_qblocks;
        s.n_slots = wgs / units > B ? wgs / units : B;
        s.chunk = MEDUSA_ATTN_MIN_CHUNK;
        s.n_splits = 0;
        s.tree_merged = 1;
        return s;
    }
    s.tile_r = 0;
    s.waves = s.rows >= kAttnLargeRows ? kAttnWavesLarge : kAttnWavesSmall;
    s.n_qblocks = (s.rows + 16 * s.waves - 1) / (16 * s.waves);
    // Split the prefix so that (a) the partial outputs (rows * d fp32 per split) stay below
    // about half the K/V bytes they summarise and (b) the grid still covers the chip when
    // there are few (sequence, kv head, query block) triples: about 1024 waves in flight.
    const int max_splits = Lcap > 0 ? (Lcap + kKeys - 1) / kKeys : 1;
    int splits = Lcap / (2 * s.rows);
    const int base = B * Hkv * s.n_qblocks;
    const int fill_blocks = 1024 / s.waves;
    const int fill = (fill_blocks + base - 1) / base;
    if (splits < fill) splits = fill;
    if (splits < 1) splits = 1;
    if (splits > max_splits) splits = max_splits;
    int chunk = Lcap > 0 ? (Lcap + splits - 1) / splits : kKeys;
    chunk = (chunk + kKeys - 1) / kKeys * kKeys;
    s.chunk = chunk;
    s.n_splits = Lcap > 0 ? (Lcap + chunk - 1) / chunk : 0;
    s.tree_merged = 0;
    s.n_slots = s.n_splits + 1;
    return s;
}

// Partial rows of the workspace: fp32 kernel [B][Hkv][slots][rows]; bf16 kernel one block
// of 32 * waves rows per workgroup.
static size_t attn_partial_rows(const AttnShape& s) {
    if (s.tile_r > 0) return (size_t)s.Hkv * s.n_slots * s.n_qblocks * (32 * s.waves);
    return (size_t)s.B * s.Hkv * s.n_slots * s.rows;
}

// bf16: byte offset of the fp32 rows that the recomputation writes (256-byte aligned)
static size_t attn_f32_rows_offset(const AttnShape& s) {
    const size_t rows = attn_partial_rows(s);
    const size_t head = rows * (size_t)s.d * 2 + rows * 4 * sizeof(float) + (size_t)s.B * 2 * sizeof(int);
    return (head + 255) / 256 * 256;
}

size_t attn_workspace_bytes(const AttnShape& s) {
    const size_t rows = attn_partial_rows(s);
    if (s.tile_r > 0)      // fp16 rows, (maximum, sum, flag, -) per row, the plan, fp32 rows
        return attn_f32_rows_offset(s) + rows * (size_t)s.d * sizeof(float);
    return rows * (size_t)s.d * sizeof(float) + rows * 2 * sizeof(float) + (size_t)s.B * 2 * sizeof(int) + 256;
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
    const size_t rows = attn_partial_rows(s);
    if (s.tile_r > 0) {
        a.ws_o = reinterpret_cast<float*>(static_cast<char*>(ws) + attn_f32_rows_offset(s));
        a.ws_h = static_cast<uint16_t*>(ws);
        a.ws_ml = reinterpret_cast<float*>(a.ws_h + rows * s.d);     // 16-byte aligned: d % 64 == 0
        a.ws_plan = reinterpret_cast<int*>(a.ws_ml + rows * 4);
    } else {
        a.ws_h = nullptr;
        a.ws_o = static_cast<float*>(ws);
        a.ws_ml = a.ws_o + rows * s.d;
        a.ws_plan = reinterpret_cast<int*>(a.ws_ml + rows * 2);
    }
    if (dt == MEDUSA_BF16) {
        return s.d == 64 ? launch_td<bf16_t, 64>(a, stream) : launch_td<bf16_t, 128>(a, stream);
    }
    return s.d == 64 ? launch_td<float, 64>(a, stream) : launch_td<float, 128>(a, stream);
}

}  // namespace medusa
