// Skinny GEMM for gfx950: Y[m, n] = sum_k X[m, k] W[n, k] with few rows m (1..64 per
// block) and many weight rows n, as in the Medusa heads (one hidden vector per head), the
// verifier's projections (one row per tree node) and the lm_head over all tree nodes.
//
// Design.  The weight matrix is the only large operand, so every workgroup streams its
// own slice of W rows from HBM exactly once, straight into MFMA operand registers: lane l
// of a wave reads 16 contiguous bytes of row (l % 16) at contraction offset 8*(l/16), so
// one load instruction covers 16 rows x 64 contiguous bytes and four unrolled k-steps
// cover 256 contiguous bytes per row.  The few X rows are staged through LDS in
// contraction chunks and re-read from there by all four waves.  The contraction runs on
// MFMA (16x16x32 bf16, or 16x16x4 fp32) with fp32 accumulation; at one row per head this
// wastes most of the matrix unit, which costs nothing because the kernel is bound by HBM.
// Epilogues are fused: bias/SiLU/residual store, per-tile top-s, or per-tile argmax.
#include "common.hpp"
#include "internal.hpp"

#include <limits.h>

namespace medusa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kLdsXBytes = 40960;     // X chunk budget (bytes of LDS)
constexpr int kSplitUnroll = 4;       // k-steps per load group in the split-contraction kernel

// Streaming-kernel tiles: RT 16-row weight tiles per wave, UN k-steps per load group.
// Chosen by a sweep on MI355X at the 8B shape (RT in {1,2,4} x UN in {2,4,8}): the
// top-s (heads) launch is flat within a few percent across the sweep, the argmax
// (verify) launch prefers short groups.
template <typename T, int EPI> struct StreamCfg { static constexpr int RT = 2, UN = 4; };
template <> struct StreamCfg<bf16_t, EPI_TOPS> { static constexpr int RT = 2, UN = 8; };
template <> struct StreamCfg<bf16_t, EPI_ARGMAX> { static constexpr int RT = 2, UN = 2; };

// acc[rt][mt][r] = Y[m0 + mt*16 + 4*lg + r][n_wave + rt*16 + ln]:
// out[m][n] = rnd(silu?(Y + bias[n]) + residual[m][n]).
template <typename T, int MT, int RT>
__device__ __forceinline__ void store_epilogue(const GemmProblem& P, const GemmBatch& bt,
                                               const floatx4 (&acc)[RT][MT], int m0, int n_wave,
                                               int ln, int lg) {
    using E = Elem<T>;
    T* out = static_cast<T*>(P.out);
    const T* bias = static_cast<const T*>(P.bias);
    const T* res = static_cast<const T*>(P.res);
    const int N = P.N;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int n = n_wave + rt * 16 + ln;
        if (n >= N) continue;
        const float bn = bias ? E::to_f32(bias[n]) : 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + mt * 16 + 4 * lg + r;
                if (m >= bt.M) continue;
                float y = acc[rt][mt][r] + bn;
                if (P.silu) y = silu(y);
                if (res) {
                    long long rr = m;
                    bool ok = true;
                    if (P.res_rows) {
                        rr = P.res_rows[m];
                        ok = rr >= 0 && rr < bt.res_rows_bound;
                    }
                    if (ok) y += E::to_f32(res[rr * P.res_stride + n]);
                }
                out[(long long)m * P.ldo + n] = E::from_f32(y);
            }
    }
}

// Problem lookup: the last problem whose first tile is <= t.
__device__ __forceinline__ int problem_of(const GemmBatch& bt, int t) {
    int pi = 0;
    while (pi + 1 < bt.n_problems && t >= bt.p[pi + 1].tile_begin) ++pi;
    return pi;
}

// Few weight rows (up to ~16K) and up to 64 input rows: all four waves of a workgroup take
// the same RT*16 weight rows and split the contraction into four contiguous quarters, so a
// small projection still spreads over hundreds of workgroups.  X fragments are read straight
// from global memory (each wave uses only its own quarter, so LDS staging would buy no
// reuse); the four partial accumulators are summed in a fixed order through LDS.
template <typename T, int MT, int RT>
__global__ __launch_bounds__(kThreads) void gemm_splitk_store_kernel(const GemmBatch bt) {
    constexpr int KS = kWaves;
    __shared__ floatx4 red[KS - 1][RT][MT][kWave];
    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    const int nblocks = bt.total_tiles * n_mb;
    const int bid = xcd_logical_block(blockIdx.x, nblocks);
    const int mb = bid % n_mb;
    const int t = bid / n_mb;
    const GemmProblem& P = bt.p[problem_of(bt, t)];
    const int tile = t - P.tile_begin;
    const int K = bt.K;
    const int N = P.N;
    const int kg = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int n_wave = tile * RT * 16;
    const int m0 = mb * MT * 16;

    const int steps = K / 32;
    const int per = (steps + KS - 1) / KS;
    const int k_lo = min(K, kg * per * 32);
    const int k_hi = min(K, (kg + 1) * per * 32);

    const T* W = static_cast<const T*>(P.W);
    const T* wrow[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        wrow[rt] = W + (long long)min(n_wave + rt * 16 + ln, N - 1) * K + 8 * lg;
    const T* X = static_cast<const T*>(P.X);
    const T* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + mt * 16 + ln;
        long long r = m;
        bool ok = m < bt.M;
        if (ok && P.x_rows) {
            r = P.x_rows[m];
            ok = r >= 0 && r < bt.x_rows_bound;
        }
        xrow[mt] = ok ? X + r * P.x_stride + 8 * lg : nullptr;
    }

    floatx4 acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto load = [&](Frag<T> (&wf)[kSplitUnroll][RT], Frag<T> (&xf)[kSplitUnroll][MT], int k) {
#pragma unroll
        for (int u = 0; u < kSplitUnroll; ++u) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) wf[u][rt].load(wrow[rt] + k + 32 * u);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (xrow[mt]) xf[u][mt].load(xrow[mt] + k + 32 * u);
                else xf[u][mt].zero();
            }
        }
    };
    auto compute = [&](const Frag<T> (&wf)[kSplitUnroll][RT], const Frag<T> (&xf)[kSplitUnroll][MT]) {
#pragma unroll
        for (int u = 0; u < kSplitUnroll; ++u)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) mma(acc[rt][mt], xf[u][mt], wf[u][rt]);
    };
    // software pipeline: group g+1's loads are in flight while group g is multiplied
    constexpr int GK = 32 * kSplitUnroll;
    const int G = (k_hi - k_lo) / GK;
    Frag<T> wa[kSplitUnroll][RT], wb[kSplitUnroll][RT];
    Frag<T> xa[kSplitUnroll][MT], xb[kSplitUnroll][MT];
    if (G > 0) load(wa, xa, k_lo);
    for (int g = 0; g < G; g += 2) {
        if (g + 1 < G) load(wb, xb, k_lo + (g + 1) * GK);
        compute(wa, xa);
        if (g + 1 < G) {
            if (g + 2 < G) load(wa, xa, k_lo + (g + 2) * GK);
            compute(wb, xb);
        }
    }
    for (int k = k_lo + G * GK; k < k_hi; k += 32) {
        Frag<T> wf[RT];
        Frag<T> xf[MT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) wf[rt].load(wrow[rt] + k);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (xrow[mt]) xf[mt].load(xrow[mt] + k);
            else xf[mt].zero();
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) mma(acc[rt][mt], xf[mt], wf[rt]);
    }

    if (kg > 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) red[kg - 1][rt][mt][lane] = acc[rt][mt];
    }
    __syncthreads();
    if (kg != 0) return;
#pragma unroll
    for (int w = 0; w < KS - 1; ++w)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[rt][mt] += red[w][rt][mt][lane];
    store_epilogue<T, MT, RT>(P, bt, acc, m0, n_wave, ln, lg);
}

// Shared epilogue of the MFMA kernels: optional fp32 logits, then the per-tile argmax or
// top-s of every input row.  acc[rt][mt][r] = Y[m0 + mt*16 + 4*lg + r][n_wave + rt*16 + ln];
// `smem` must hold Mb * NWG floats (top-s only) and may alias the kernel's X staging area.
template <int MT, int RT, int NWG, int EPI>
__device__ __forceinline__ void tile_epilogue(const GemmProblem& P, const GemmBatch& bt,
                                              const floatx4 (&acc)[RT][MT], int m0, int Mb,
                                              int tile, int n_wave, int wave, int lane,
                                              unsigned char* smem, float (&red_v)[kWaves][MT * 16],
                                              int (&red_i)[kWaves][MT * 16]) {
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int N = P.N;
    if (P.logits) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int n = n_wave + rt * 16 + ln;
            if (n >= N) continue;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + mt * 16 + 4 * lg + r;
                    if (m < bt.M) P.logits[(long long)m * P.logits_ld + n] = acc[rt][mt][r];
                }
        }
    }

    if (EPI == EPI_ARGMAX) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float bv = -INFINITY;
                int bi = INT_MAX;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const int n = n_wave + rt * 16 + ln;
                    const float v = n < N ? acc[rt][mt][r] : -INFINITY;
                    const int i = n < N ? n : INT_MAX;
                    if (better(v, i, bv, bi)) { bv = v; bi = i; }
                }
                row_best(bv, bi);
                if (ln == 0) {
                    red_v[wave][mt * 16 + 4 * lg + r] = bv;
                    red_i[wave][mt * 16 + 4 * lg + r] = bi;
                }
            }
        __syncthreads();
        for (int m = threadIdx.x; m < Mb; m += kThreads) {
            float bv = red_v[0][m];
            int bi = red_i[0][m];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                if (better(red_v[w][m], red_i[w][m], bv, bi)) { bv = red_v[w][m]; bi = red_i[w][m]; }
            const long long o = (long long)(m0 + m) * P.n_tiles + tile;
            P.part_val[o] = bv;
            P.part_idx[o] = bi;
        }
        return;
    }

    if (EPI == EPI_TOPS) {
        // Only MT == 1 (<= 16 rows) is instantiated for this epilogue.
        __syncthreads();
        float* sv = reinterpret_cast<float*>(smem);      // [Mb][NWG]
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int nl = wave * RT * 16 + rt * 16 + ln;
            const int n = tile * NWG + nl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * lg + r;
                if (m < Mb) sv[m * NWG + nl] = n < N ? acc[rt][0][r] : -INFINITY;
            }
        }
        __syncthreads();
        constexpr int PER = NWG / kWave;
        const int s = P.s;
        for (int m = wave; m < Mb; m += kWaves) {
            float v[PER];
            int id[PER];
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int nl = lane + kWave * j;
                const int n = tile * NWG + nl;
                v[j] = n < N ? sv[m * NWG + nl] : -INFINITY;
                id[j] = n < N ? n : INT_MAX;
            }
            const long long o = ((long long)(m0 + m) * P.n_tiles + tile) * s;
            for (int round = 0; round < s; ++round) {
                float bv = v[0];
                int bi = id[0];
#pragma unroll
                for (int j = 1; j < PER; ++j)
                    if (better(v[j], id[j], bv, bi)) { bv = v[j]; bi = id[j]; }
                wave_best(bv, bi);
                if (lane == 0) {
                    P.part_val[o + round] = bv;
                    P.part_idx[o + round] = bi;
                }
#pragma unroll
                for (int j = 0; j < PER; ++j)
                    if (id[j] == bi) { v[j] = -INFINITY; id[j] = INT_MAX; }
            }
        }
    }
}

template <typename T, int MT, int RT, int UN, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const GemmBatch bt) {
    using E = Elem<T>;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red_v[kWaves][MT * 16];
    __shared__ int red_i[kWaves][MT * 16];

    constexpr int NWG = kWaves * RT * 16;
    constexpr int EPV = 16 / sizeof(T);     // elements per 16-byte vector
    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    const int nblocks = bt.total_tiles * n_mb;
    const int bid = xcd_logical_block(blockIdx.x, nblocks);
    const int mb = bid % n_mb;
    const int t = bid / n_mb;
    const GemmProblem& P = bt.p[problem_of(bt, t)];
    const int tile = t - P.tile_begin;
    const int K = bt.K;
    const int N = P.N;

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int n_wave = tile * NWG + wave * RT * 16;
    const int m0 = mb * MT * 16;
    const int Mb = min(bt.M - m0, MT * 16);

    const T* W = static_cast<const T*>(P.W);
    const T* wrow[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        int n = min(n_wave + rt * 16 + ln, N - 1);
        wrow[rt] = W + (long long)n * K + 8 * lg;
    }

    floatx4 acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    T* xs = reinterpret_cast<T*>(smem);
    const int KC = bt.KC;               // a multiple of 32 * UN unless K is smaller
    const int pitch = KC + 8;
    const T* X = static_cast<const T*>(P.X);
    int kc_staged = -1;

    // Stage X[m0 .. m0+Mb)[kc .. kc+KC) into LDS (all threads; uniform call).
    auto stage = [&](int kc) {
        __syncthreads();
        const int klen = min(KC, K - kc);
        const int per_row = klen / EPV;
        for (int idx = threadIdx.x; idx < Mb * per_row; idx += kThreads) {
            const int m = idx / per_row;
            const int c = idx - m * per_row;
            const int row = m0 + m;
            long long r = row;
            bool ok = true;
            if (P.x_rows) {
                r = P.x_rows[row];
                ok = r >= 0 && r < bt.x_rows_bound;
            }
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (ok) v = *reinterpret_cast<const u32x4*>(X + r * P.x_stride + kc + c * EPV);
            *reinterpret_cast<u32x4*>(xs + m * pitch + c * EPV) = v;
        }
        __syncthreads();
        kc_staged = kc;
    };
    auto load_w = [&](Frag<T> (&wf)[UN][RT], int k) {
#pragma unroll
        for (int u = 0; u < UN; ++u)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) wf[u][rt].load(wrow[rt] + k + 32 * u);
    };
    auto compute = [&](const Frag<T> (&wf)[UN][RT], int k) {
        const int c = k / KC * KC;
        if (c != kc_staged) stage(c);
        const int kl = k - c;
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            Frag<T> xf[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = mt * 16 + ln;
                if (m < Mb) xf[mt].load(xs + m * pitch + kl + 32 * u + 8 * lg);
                else xf[mt].zero();
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) mma(acc[rt][mt], xf[mt], wf[u][rt]);
        }
    };

    // Software pipeline over groups of UN k-steps: the W loads of group g+1 are in
    // flight while group g is multiplied.
    constexpr int GK = 32 * UN;
    const int G = K / GK;
    Frag<T> wa[UN][RT], wb[UN][RT];
    if (G > 0) load_w(wa, 0);
    for (int g = 0; g < G; g += 2) {
        if (g + 1 < G) load_w(wb, (g + 1) * GK);
        compute(wa, g * GK);
        if (g + 1 < G) {
            if (g + 2 < G) load_w(wa, (g + 2) * GK);
            compute(wb, (g + 1) * GK);
        }
    }
    for (int k = G * GK; k < K; k += 32) {
        const int c = k / KC * KC;
        if (c != kc_staged) stage(c);
        Frag<T> wf[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) wf[rt].load(wrow[rt] + k);
        Frag<T> xf[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + ln;
            if (m < Mb) xf[mt].load(xs + m * pitch + (k - c) + 8 * lg);
            else xf[mt].zero();
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) mma(acc[rt][mt], xf[mt], wf[rt]);
    }

    // acc[rt][mt][r] = Y[m0 + mt*16 + 4*lg + r][n_wave + rt*16 + ln]
    if (EPI == EPI_STORE) {
        store_epilogue<T, MT, RT>(P, bt, acc, m0, n_wave, ln, lg);
        return;
    }

    tile_epilogue<MT, RT, NWG, EPI>(P, bt, acc, m0, Mb, tile, n_wave, wave, lane, smem, red_v, red_i);
}

// Row-streaming MFMA kernel (bf16; lm_head over the tree nodes, heads at batch > 2).
// Each wave owns 16*RT weight rows and streams them in contraction chunks with
// row-contiguous non-temporal loads (one instruction = 64 lanes x 16 contiguous bytes
// spread over as many rows as the chunk requires), close to the access pattern that
// reaches 7.0 TB/s.  The chunk is transposed through a wave-private
// LDS tile into the MFMA operand layout (row l%16, k-slot 8*(l/16)); the X rows of the
// chunk are staged once per workgroup and shared by the four waves.  The next chunk's
// weights are in flight in registers while the current one is multiplied.
// Chosen by a sweep at the 8B shape (lm_head over 64 nodes): chunk 64 / 4 tiles per wave
// 161 us, 128 / 2: 172 us, 256 / 1: 236 us (the smaller chunk keeps LDS per workgroup low
// enough for more workgroups per CU).
#ifndef MEDUSA_RS_CHUNK
#define MEDUSA_RS_CHUNK 64
#endif
#ifndef MEDUSA_RS_RTW
#define MEDUSA_RS_RTW 4
#endif
constexpr int kRsChunk = MEDUSA_RS_CHUNK;   // contraction chunk per pass
constexpr int kRsRtw = MEDUSA_RS_RTW;       // 16-row weight tiles per wave (argmax, top-s)
constexpr int kRsRtwPartial = 1;            // ... for contraction slices (small weights)

template <int MT, int EPI, int RTW>
__global__ __launch_bounds__(kThreads) void gemm_rowstream_kernel(const GemmBatch bt) {
    constexpr int RT = RTW;
    constexpr int ROWS = 16 * RT;             // weight rows per wave
    constexpr int NWG = kWaves * ROWS;
    constexpr int XP = kRsChunk + 8;          // LDS pitch of X rows and W tiles (elements)
    constexpr int LPR = kRsChunk / 8;         // lanes per row in one load instruction
    constexpr int RPI = kWave / LPR;          // rows per load instruction
    constexpr int NI = ROWS / RPI;            // 16-byte loads per lane per chunk
    __shared__ __align__(16) bf16_t xs[MT * 16 * XP];
    __shared__ __align__(16) bf16_t wt[kWaves][ROWS * XP];
    __shared__ float red_v[kWaves][MT * 16];
    __shared__ int red_i[kWaves][MT * 16];

    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    const int nks = EPI == EPI_PARTIAL ? bt.ksplit : 1;
    const int nblocks = bt.total_tiles * n_mb * nks;
    int bid = xcd_logical_block(blockIdx.x, nblocks);
    const int mb = bid % n_mb;
    bid /= n_mb;
    const int ksl = bid % nks;
    const int t = bid / nks;
    const GemmProblem& P = bt.p[problem_of(bt, t)];
    const int tile = t - P.tile_begin;
    const int K = bt.K;
    const int N = P.N;
    // contraction slice of this block (whole chunks)
    const int chunks = K / kRsChunk;
    const int per = (chunks + nks - 1) / nks;
    const int k_lo = min(K, ksl * per * kRsChunk);
    const int k_hi = min(K, (ksl + 1) * per * kRsChunk);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int n_wave = tile * NWG + wave * ROWS;
    const int m0 = mb * MT * 16;
    const int Mb = min(bt.M - m0, MT * 16);

    // load i covers rows RPI*i .. RPI*i+RPI-1 of the wave's rows, LPR lanes per row
    const bf16_t* W = static_cast<const bf16_t*>(P.W);
    const int half = lane / LPR;
    const int col = (lane % LPR) * 8;
    const u32x4* wsrc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int n = min(n_wave + RPI * i + half, N - 1);
        wsrc[i] = reinterpret_cast<const u32x4*>(W + (long long)n * K + col);
    }
    u32x4 wr[NI];
    auto load_w = [&](int kc) {
#pragma unroll
        for (int i = 0; i < NI; ++i) wr[i] = __builtin_nontemporal_load(wsrc[i] + kc / 8);
    };
    const bf16_t* X = static_cast<const bf16_t*>(P.X);
    bf16_t* wtile = wt[wave];

    floatx4 acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // X rows of the chunk are fetched one chunk ahead as well (XV vectors per thread)
    constexpr int VPR = kRsChunk / 8;                       // 16-byte vectors per X row chunk
    constexpr int XV = (MT * 16 * VPR + kThreads - 1) / kThreads;
    const bf16_t* xrow_ptr[XV];
    int xdst[XV];
#pragma unroll
    for (int j = 0; j < XV; ++j) {
        const int idx = threadIdx.x + j * kThreads;
        const int m = idx / VPR;
        const int c = idx - m * VPR;
        xdst[j] = -1;
        xrow_ptr[j] = nullptr;
        if (m < Mb) {
            long long r = m0 + m;
            bool ok = true;
            if (P.x_rows) {
                r = P.x_rows[m0 + m];
                ok = r >= 0 && r < bt.x_rows_bound;
            }
            xdst[j] = m * XP + c * 8;
            if (ok) xrow_ptr[j] = X + r * P.x_stride + c * 8;
        }
    }
    u32x4 xr[XV];
    auto load_x = [&](int kc) {
#pragma unroll
        for (int j = 0; j < XV; ++j)
            xr[j] = xrow_ptr[j] ? *reinterpret_cast<const u32x4*>(xrow_ptr[j] + kc)
                                : u32x4{0u, 0u, 0u, 0u};
    };

    if (k_lo < k_hi) {
        load_w(k_lo);
        load_x(k_lo);
    }
    for (int kc = k_lo; kc < k_hi; kc += kRsChunk) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < XV; ++j)
            if (xdst[j] >= 0) *reinterpret_cast<u32x4*>(xs + xdst[j]) = xr[j];
#pragma unroll
        for (int i = 0; i < NI; ++i)
            *reinterpret_cast<u32x4*>(wtile + (RPI * i + half) * XP + col) = wr[i];
        __syncthreads();
        if (kc + kRsChunk < k_hi) {
            load_w(kc + kRsChunk);
            load_x(kc + kRsChunk);
        }
#pragma unroll
        for (int ks = 0; ks < kRsChunk; ks += 32) {
            Frag<bf16_t> wf[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) wf[rt].load(wtile + (rt * 16 + ln) * XP + ks + 8 * lg);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                Frag<bf16_t> xf;
                const int m = mt * 16 + ln;
                if (m < Mb) xf.load(xs + m * XP + ks + 8 * lg);
                else xf.zero();
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) mma(acc[rt][mt], xf, wf[rt]);
            }
        }
    }
    if (EPI == EPI_PARTIAL) {
        float* part = P.part_val + (long long)ksl * bt.M * N;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int n = n_wave + rt * 16 + ln;
            if (n >= N) continue;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + mt * 16 + 4 * lg + r;
                    if (m < bt.M) part[(long long)m * N + n] = acc[rt][mt][r];
                }
        }
        return;
    }
    // the top-s epilogue needs Mb * NWG floats of scratch: the W tiles are free by now
    static_assert(EPI != EPI_TOPS || sizeof(wt) >= 16 * NWG * sizeof(float), "top-s scratch");
    __syncthreads();
    tile_epilogue<MT, RT, NWG, EPI>(P, bt, acc, m0, Mb, tile, n_wave, wave, lane,
                                    reinterpret_cast<unsigned char*>(&wt[0][0]), red_v, red_i);
}

// Sum the contraction slices of every (m, n) in slice order and apply the store epilogue:
// out[m][n] = rnd(silu?(sum + bias[n]) + residual[m][n]).  Four consecutive n per thread.
template <typename T>
__global__ __launch_bounds__(kThreads) void splitk_finalize_kernel(const GemmBatch bt) {
    using E = Elem<T>;
    long long q = (long long)blockIdx.x * kThreads + threadIdx.x;     // quad index
    int pi = 0;
    for (; pi < bt.n_problems; ++pi) {
        const long long nq = (long long)bt.M * ((bt.p[pi].N + 3) / 4);
        if (q < nq) break;
        q -= nq;
    }
    if (pi >= bt.n_problems) return;
    const GemmProblem& P = bt.p[pi];
    const int N = P.N;
    const int qpr = (N + 3) / 4;
    const int m = (int)(q / qpr);
    const int n0 = (int)(q - (long long)m * qpr) * 4;
    float y[4] = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < bt.ksplit; ++ks) {
        const float* part = P.part_val + ((long long)ks * bt.M + m) * N;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (n0 + j < N) y[j] += part[n0 + j];
    }
    const T* bias = static_cast<const T*>(P.bias);
    const T* res = static_cast<const T*>(P.res);
    long long rr = m;
    bool rok = res != nullptr;
    if (rok && P.res_rows) {
        rr = P.res_rows[m];
        rok = rr >= 0 && rr < bt.res_rows_bound;
    }
    T* out = static_cast<T*>(P.out);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + j;
        if (n >= N) continue;
        float v = y[j] + (bias ? E::to_f32(bias[n]) : 0.f);
        if (P.silu) v = silu(v);
        if (rok) v += E::to_f32(res[rr * P.res_stride + n]);
        out[(long long)m * P.ldo + n] = E::from_f32(v);
    }
}

// GEMV for one or two input rows (the heads and the bootstrap root at batch 1): every
// wave streams whole weight rows with row-contiguous, non-temporal 16-byte loads (64 lanes
// cover 1 KiB of one row per instruction), which measured 7.0 TB/s on MI355X against
// 6.2 TB/s for plain loads and 5.3 TB/s for the MFMA operand pattern.  At one or two rows
// the dot products fit the vector ALU (v_dot2_f32_bf16, two MACs per lane per instruction,
// about 6 % of issue at full bandwidth), so no MFMA and no transposition are needed.
// Lane l keeps X[m][512 c + 8 l .. +8] of every 512-wide chunk c in registers; a row's
// partial sums are reduced across the wave in a fixed order.  Results go to LDS and the
// same epilogues as the MFMA kernels run on them (per-tile top-s, or bias/SiLU/residual
// store), with the same tiles (128 rows for top-s, 32 for the store).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8(const u32x4& w, const u32x4& x, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // copy the lanes out first: bit-casting a vector-element lvalue directly made the
        // compiler read element 0 for every i
        const uint32_t wi = w[i];
        const uint32_t xi = x[i];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wi),
                                              __builtin_bit_cast(bf16x2_t, xi), acc, false);
    }
    return acc;
}

template <int NCH, int MV, int R, int EPI>
__global__ __launch_bounds__(kThreads) void gemv_bf16_kernel(const GemmBatch bt) {
    constexpr int RPW = EPI == EPI_TOPS ? 32 : 8;      // weight rows per wave
    constexpr int NWG = kWaves * RPW;
    __shared__ float yl[MV][NWG];
    const int n_mb = (bt.M + MV - 1) / MV;
    const int nblocks = bt.total_tiles * n_mb;
    const int bid = xcd_logical_block(blockIdx.x, nblocks);
    const int mb = bid % n_mb;
    const int t = bid / n_mb;
    const GemmProblem& P = bt.p[problem_of(bt, t)];
    const int tile = t - P.tile_begin;
    const int K = bt.K;
    const int N = P.N;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int m0 = mb * MV;
    const int Mb = min(bt.M - m0, MV);

    const bf16_t* X = static_cast<const bf16_t*>(P.X);
    u32x4 xs[MV][NCH];
#pragma unroll
    for (int mv = 0; mv < MV; ++mv) {
        long long r = m0 + mv;
        bool ok = mv < Mb;
        if (ok && P.x_rows) {
            r = P.x_rows[m0 + mv];
            ok = r >= 0 && r < bt.x_rows_bound;
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            xs[mv][c] = ok ? *reinterpret_cast<const u32x4*>(X + r * P.x_stride + c * 512 + 8 * lane)
                           : u32x4{0u, 0u, 0u, 0u};
    }

    const bf16_t* W = static_cast<const bf16_t*>(P.W);
    const int n_wave = tile * NWG + wave * RPW;
    auto load = [&](u32x4 (&w)[R][NCH], int j) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = min(n_wave + j + r, N - 1);
            const u32x4* row = reinterpret_cast<const u32x4*>(W + (long long)n * K) + lane;
#pragma unroll
            for (int c = 0; c < NCH; ++c) w[r][c] = __builtin_nontemporal_load(row + c * 64);
        }
    };
    auto compute = [&](const u32x4 (&w)[R][NCH], int j) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int mv = 0; mv < MV; ++mv) {
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < NCH; ++c) acc = dot8(w[r][c], xs[mv][c], acc);
                acc = wave_sum_dpp(acc);
                if (lane == 0) yl[mv][wave * RPW + j + r] = acc;
            }
    };
    u32x4 wa[R][NCH], wb[R][NCH];
    load(wa, 0);
    for (int j = 0; j < RPW; j += 2 * R) {
        if (j + R < RPW) load(wb, j + R);
        compute(wa, j);
        if (j + R < RPW) {
            if (j + 2 * R < RPW) load(wa, j + 2 * R);
            compute(wb, j + R);
        }
    }
    __syncthreads();

    if (EPI == EPI_STORE) {
        using E = Elem<bf16_t>;
        bf16_t* out = static_cast<bf16_t*>(P.out);
        const bf16_t* bias = static_cast<const bf16_t*>(P.bias);
        const bf16_t* res = static_cast<const bf16_t*>(P.res);
        for (int idx = threadIdx.x; idx < Mb * NWG; idx += kThreads) {
            const int mv = idx / NWG;
            const int nl = idx - mv * NWG;
            const int n = tile * NWG + nl;
            if (n >= N) continue;
            const int m = m0 + mv;
            float y = yl[mv][nl] + (bias ? E::to_f32(bias[n]) : 0.f);
            if (P.silu) y = silu(y);
            if (res) {
                long long rr = m;
                bool ok = true;
                if (P.res_rows) {
                    rr = P.res_rows[m];
                    ok = rr >= 0 && rr < bt.res_rows_bound;
                }
                if (ok) y += E::to_f32(res[rr * P.res_stride + n]);
            }
            out[(long long)m * P.ldo + n] = E::from_f32(y);
        }
        return;
    }

    // EPI_TOPS
    if (P.logits) {
        for (int idx = threadIdx.x; idx < Mb * NWG; idx += kThreads) {
            const int mv = idx / NWG;
            const int nl = idx - mv * NWG;
            const int n = tile * NWG + nl;
            if (n < N) P.logits[(long long)(m0 + mv) * P.logits_ld + n] = yl[mv][nl];
        }
    }
    constexpr int PER = NWG >= kWave ? NWG / kWave : 1;   // the top-s tiles are 128 rows
    const int s = P.s;
    for (int mv = wave; mv < Mb; mv += kWaves) {
        float v[PER];
        int id[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int nl = lane + kWave * j;
            const int n = tile * NWG + nl;
            v[j] = n < N ? yl[mv][nl] : -INFINITY;
            id[j] = n < N ? n : INT_MAX;
        }
        const long long o = ((long long)(m0 + mv) * P.n_tiles + tile) * s;
        for (int round = 0; round < s; ++round) {
            float bv = v[0];
            int bi = id[0];
#pragma unroll
            for (int j = 1; j < PER; ++j)
                if (better(v[j], id[j], bv, bi)) { bv = v[j]; bi = id[j]; }
            wave_best(bv, bi);
            if (lane == 0) {
                P.part_val[o + round] = bv;
                P.part_idx[o + round] = bi;
            }
#pragma unroll
            for (int j = 0; j < PER; ++j)
                if (id[j] == bi) { v[j] = -INFINITY; id[j] = INT_MAX; }
        }
    }
}

// Merge of the per-tile candidate lists (each sorted best first) into the top-s, in the
// (value desc, id asc) order of `better`.
//  1. Each thread holds the first entries (tile maxima) of tiles tid + 256 j.
//  2. Lower bound tau on the s-th best tile maximum: in each wave the s-th best of the 64
//     lane maxima is reached by s distinct tiles, so it is <= the s-th best overall; tau is
//     the best of the four wave bounds.
//  3. Tiles whose maximum is >= tau are compacted.  A wave contributes only from its s lanes
//     at or above its own bound, so there are at most 4 * s * kMergeSlots of them.
//  4. Their ranks by counting; rank r < s names the r-th best tile.
//  5. Entry j of the r-th best tile has at least r + j better entries (the first entries of
//     the r better tiles and j entries of its own list), so only r + j < s can reach the
//     top-s, and no entry of any other tile can: s (s + 1) / 2 candidates.
//  6. Their ranks by counting; rank < s is the output slot.
// Each selection is one pass of independent comparisons instead of s dependent rounds, and
// a comparison is one unsigned 64-bit compare of packed keys (merge_key).
constexpr int kMergeSlots = 8;
constexpr int kMergeMaxTiles = kThreads * kMergeSlots;
constexpr int kMergeStep3 = kWaves * MEDUSA_MAX_TOPK * kMergeSlots;
constexpr int kMergeStep5 = MEDUSA_MAX_TOPK * (MEDUSA_MAX_TOPK + 1) / 2;
constexpr int kMergeMaxCand = kMergeStep3 > kMergeStep5 ? kMergeStep3 : kMergeStep5;

// (value, id) as one key whose unsigned order is the `better` order: the high word is the
// value's bits mapped so that unsigned order is float order (-0 folded onto +0), the low
// word the complement of the id (lower id = larger word).  Real pairs are distinct.  Padding
// (id INT_MAX, value -inf) gets a distinct low word per slot, below every real id's.
constexpr uint32_t kOrdNegInf = 0x007FFFFFu;    // order word of -inf (0xFF800000)
__device__ __forceinline__ uint64_t merge_key(float v, int id, int slot) {
    if (id == INT_MAX) return ((uint64_t)kOrdNegInf << 32) | (uint32_t)(0x7FFFFFFF - slot);
    const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ bool merge_key_is_pad(uint64_t k) { return (uint32_t)k < 0x80000000u; }
__device__ __forceinline__ int merge_key_id(uint64_t k) {
    return merge_key_is_pad(k) ? -1 : (int)(0xFFFFFFFFu - (uint32_t)k);
}
__device__ __forceinline__ float merge_key_value(uint64_t k) {
    const uint32_t o = (uint32_t)(k >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Number of keys[0, n) greater than k.
__device__ __forceinline__ int key_rank(const uint64_t* keys, int n, uint64_t k) {
    int r = 0;
#pragma unroll 8
    for (int c = 0; c < n; ++c) r += keys[c] > k ? 1 : 0;
    return r;
}

__global__ __launch_bounds__(kThreads) void topk_merge_kernel(const MergeBatch bt) {
    __shared__ uint64_t cand[kMergeMaxCand];
    __shared__ int cand_tile[kMergeStep3];
    __shared__ uint64_t lane_best[kThreads];
    __shared__ uint64_t wave_bound[kWaves];
    __shared__ int best_tiles[MEDUSA_MAX_TOPK];
    __shared__ int n_cand, n_cand2;
    const int p = blockIdx.x / bt.M;
    const int m = blockIdx.x - p * bt.M;
    const MergeProblem& P = bt.p[p];
    const int s = P.s;
    const int nt = P.n_tiles;
    const float* pv = P.part_val + (long long)m * nt * s;
    const int32_t* pi = P.part_idx + (long long)m * nt * s;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;

    // 1. tile maxima; slots past n_tiles are padding
    uint64_t key[kMergeSlots];
#pragma unroll
    for (int j = 0; j < kMergeSlots; ++j) {
        const int t = tid + kThreads * j;
        const float v = t < nt ? pv[(long long)t * s] : -INFINITY;
        const int id = t < nt ? pi[(long long)t * s] : INT_MAX;
        key[j] = merge_key(v, id, t);
    }
    if (tid == 0) { n_cand = 0; n_cand2 = 0; }
    // 2. lane maximum, its rank within the wave, the wave bound
    uint64_t lb = key[0];
#pragma unroll
    for (int j = 1; j < kMergeSlots; ++j) lb = key[j] > lb ? key[j] : lb;
    lane_best[tid] = lb;
    __syncthreads();
    if (key_rank(lane_best + wave * kWave, kWave, lb) == s - 1) wave_bound[wave] = lb;
    __syncthreads();
    uint64_t tau = wave_bound[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) tau = wave_bound[w] > tau ? wave_bound[w] : tau;
    // 3. compaction of the tiles at or above tau
#pragma unroll
    for (int j = 0; j < kMergeSlots; ++j) {
        if (key[j] >= tau) {
            const int c = atomicAdd(&n_cand, 1);
            cand[c] = key[j];
            cand_tile[c] = tid + kThreads * j;
        }
    }
    __syncthreads();
    // 4. the s best tiles (padding slots name no tile)
    const int nc = n_cand;
    for (int c = tid; c < nc; c += kThreads) {
        const int r = key_rank(cand, nc, cand[c]);
        if (r < s) best_tiles[r] = cand_tile[c] < nt ? cand_tile[c] : -1;
    }
    __syncthreads();
    // 5. entries (r, j) with r + j < s of those tiles
    for (int c = tid; c < s * s; c += kThreads) {
        const int r = c / s;
        const int j = c - r * s;
        const int t = best_tiles[r];
        if (j < s - r && t >= 0) {
            const uint64_t k = merge_key(pv[(long long)t * s + j], pi[(long long)t * s + j], c);
            cand[atomicAdd(&n_cand2, 1)] = k;
        }
    }
    __syncthreads();
    // 6. the top-s of those, in order
    const int nc2 = n_cand2;
    for (int c = tid; c < nc2; c += kThreads) {
        const uint64_t k = cand[c];
        const int r = key_rank(cand, nc2, k);
        if (r < s) {
            P.out_ids[(long long)m * P.out_ld + r] = merge_key_id(k);
            if (P.out_vals) P.out_vals[(long long)m * P.out_ld + r] = merge_key_is_pad(k) ? -INFINITY : merge_key_value(k);
        }
    }
    // fewer than s candidates (vocabularies smaller than s): the rest are padding
    for (int r = nc2 + tid; r < s; r += kThreads) {
        P.out_ids[(long long)m * P.out_ld + r] = -1;
        if (P.out_vals) P.out_vals[(long long)m * P.out_ld + r] = -INFINITY;
    }
    for (int r = s + tid; r < P.s_pad; r += kThreads) {
        P.out_ids[(long long)m * P.out_ld + r] = -1;
        if (P.out_vals) P.out_vals[(long long)m * P.out_ld + r] = 0.f;
    }
}

template <typename T, int MT, int EPI>
hipError_t launch_t(GemmBatch& bt, hipStream_t stream) {
    constexpr int RT = StreamCfg<T, EPI>::RT;
    constexpr int UN = StreamCfg<T, EPI>::UN;
    const int mrows = min(bt.M, MT * 16);
    constexpr int GK = 32 * UN;
    int kc = (kLdsXBytes / (mrows * (int)sizeof(T)) - 8) / GK * GK;
    kc = max(GK, min(kc, (bt.K + GK - 1) / GK * GK));
    bt.KC = kc;
    size_t lds = (size_t)mrows * (kc + 8) * sizeof(T);
    if (EPI == EPI_TOPS) {
        const size_t need = (size_t)mrows * kWaves * RT * 16 * sizeof(float);
        if (need > lds) lds = need;
    }
    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    dim3 grid(bt.total_tiles * n_mb);
    hipLaunchKernelGGL((gemm_kernel<T, MT, RT, UN, EPI>), grid, dim3(kThreads), lds, stream, bt);
    return hipGetLastError();
}

template <typename T, int MT, int RT>
hipError_t launch_splitk(GemmBatch& bt, hipStream_t stream) {
    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    hipLaunchKernelGGL((gemm_splitk_store_kernel<T, MT, RT>), dim3(bt.total_tiles * n_mb),
                       dim3(kThreads), 0, stream, bt);
    return hipGetLastError();
}

// Weight rows per workgroup of the split-contraction store kernel.
int splitk_rt(int M) { return M <= 16 ? 2 : 1; }

template <typename T>
hipError_t launch_store(GemmBatch& bt, hipStream_t stream) {
    if (bt.M <= 16) return launch_splitk<T, 1, 2>(bt, stream);
    if (bt.M <= 32) return launch_splitk<T, 2, 1>(bt, stream);
    return launch_splitk<T, 4, 1>(bt, stream);
}

template <typename T, int EPI>
hipError_t launch_mt(GemmBatch& bt, hipStream_t stream) {
    if (EPI == EPI_TOPS || bt.M <= 16) return launch_t<T, 1, EPI>(bt, stream);
    if (bt.M <= 32) return launch_t<T, 2, EPI>(bt, stream);
    return launch_t<T, 4, EPI>(bt, stream);
}

template <typename T>
hipError_t launch_epi(int epi, GemmBatch& bt, hipStream_t stream) {
    switch (epi) {
        case EPI_STORE: return launch_store<T>(bt, stream);
        case EPI_TOPS: return launch_mt<T, EPI_TOPS>(bt, stream);
        default: return launch_mt<T, EPI_ARGMAX>(bt, stream);
    }
}

}  // namespace

bool rowstream_eligible(medusa_dtype dt, int epi, int M, int K);

int gemm_rows_per_tile(medusa_dtype dt, int M, int epi, int K) {
    if (epi == EPI_STORE) return 16 * splitk_rt(M);
    if (epi == EPI_PARTIAL) return kWaves * 16 * kRsRtwPartial;
    if (rowstream_eligible(dt, epi, M, K)) return kWaves * 16 * kRsRtw;
    int rt;
    if (dt == MEDUSA_BF16)
        rt = epi == EPI_TOPS ? StreamCfg<bf16_t, EPI_TOPS>::RT : StreamCfg<bf16_t, EPI_ARGMAX>::RT;
    else
        rt = epi == EPI_TOPS ? StreamCfg<float, EPI_TOPS>::RT : StreamCfg<float, EPI_ARGMAX>::RT;
    return kWaves * 16 * rt;
}

namespace {

template <int NCH, int MV, int EPI>
hipError_t launch_gemv(GemmBatch& bt, hipStream_t stream) {
    const int n_mb = (bt.M + MV - 1) / MV;
    hipLaunchKernelGGL((gemv_bf16_kernel<NCH, MV, 1, EPI>), dim3(bt.total_tiles * n_mb),
                       dim3(kThreads), 0, stream, bt);
    return hipGetLastError();
}

template <int NCH, int EPI>
hipError_t launch_gemv_m(GemmBatch& bt, hipStream_t stream) {
    return bt.M == 1 ? launch_gemv<NCH, 1, EPI>(bt, stream) : launch_gemv<NCH, 2, EPI>(bt, stream);
}

template <int EPI>
hipError_t launch_gemv_k(GemmBatch& bt, hipStream_t stream) {
    switch (bt.K / 512) {
        case 1: return launch_gemv_m<1, EPI>(bt, stream);
        case 2: return launch_gemv_m<2, EPI>(bt, stream);
        case 4: return launch_gemv_m<4, EPI>(bt, stream);
        case 8: return launch_gemv_m<8, EPI>(bt, stream);
        default: return launch_gemv_m<16, EPI>(bt, stream);
    }
}

// The streaming GEMV path serves bf16 with at most two input rows and a contraction that
// is a multiple of 512 up to 8192 (one to sixteen 1 KiB chunks per row).
bool gemv_eligible(medusa_dtype dt, int epi, const GemmBatch& bt) {
    if (dt != MEDUSA_BF16 || bt.M > 2 || bt.K % 512 != 0) return false;
    const int nch = bt.K / 512;
    if (nch != 1 && nch != 2 && nch != 4 && nch != 8 && nch != 16) return false;
    return epi == EPI_TOPS || epi == EPI_STORE;
}

}  // namespace

template <int MT, int EPI, int RTW>
hipError_t launch_rowstream_t(GemmBatch& bt, hipStream_t stream) {
    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    const int nks = EPI == EPI_PARTIAL ? bt.ksplit : 1;
    hipLaunchKernelGGL((gemm_rowstream_kernel<MT, EPI, RTW>), dim3(bt.total_tiles * n_mb * nks),
                       dim3(kThreads), 0, stream, bt);
    return hipGetLastError();
}

hipError_t launch_rowstream(int epi, GemmBatch& bt, hipStream_t stream) {
    if (epi == EPI_TOPS) return launch_rowstream_t<1, EPI_TOPS, kRsRtw>(bt, stream);
    if (epi == EPI_PARTIAL) {
        if (bt.M <= 16) return launch_rowstream_t<1, EPI_PARTIAL, kRsRtwPartial>(bt, stream);
        if (bt.M <= 32) return launch_rowstream_t<2, EPI_PARTIAL, kRsRtwPartial>(bt, stream);
        return launch_rowstream_t<4, EPI_PARTIAL, kRsRtwPartial>(bt, stream);
    }
    if (bt.M <= 16) return launch_rowstream_t<1, EPI_ARGMAX, kRsRtw>(bt, stream);
    if (bt.M <= 32) return launch_rowstream_t<2, EPI_ARGMAX, kRsRtw>(bt, stream);
    return launch_rowstream_t<4, EPI_ARGMAX, kRsRtw>(bt, stream);
}

// Row-streaming MFMA path: bf16, contraction a multiple of its 256-wide chunk, argmax or
// top-s epilogue (top-s only past the GEMV's two rows).
bool rowstream_eligible(medusa_dtype dt, int epi, int M, int K) {
    if (dt != MEDUSA_BF16 || K % kRsChunk != 0) return false;
    return epi == EPI_ARGMAX || (epi == EPI_TOPS && M > 2);
}

int store_ksplit(medusa_dtype dt, int M, int K, int tiles) {
    if (dt != MEDUSA_BF16 || M <= 16 || K % kRsChunk != 0) return 0;
    const int n_mb = (M + 63) / 64;
    const int want = (384 + tiles * n_mb - 1) / (tiles * n_mb);   // about 384 workgroups
    return max(1, min(want, min(8, K / kRsChunk)));
}

hipError_t gemm_store_partial_launch(medusa_dtype dt, GemmBatch& bt, hipStream_t stream) {
    hipError_t e = launch_rowstream(EPI_PARTIAL, bt, stream);
    if (e != hipSuccess) return e;
    long long quads = 0;
    for (int p = 0; p < bt.n_problems; ++p) quads += (long long)bt.M * ((bt.p[p].N + 3) / 4);
    const int blocks = (int)((quads + kThreads - 1) / kThreads);
    if (dt == MEDUSA_BF16)
        hipLaunchKernelGGL(splitk_finalize_kernel<bf16_t>, dim3(blocks), dim3(kThreads), 0, stream, bt);
    else
        hipLaunchKernelGGL(splitk_finalize_kernel<float>, dim3(blocks), dim3(kThreads), 0, stream, bt);
    return hipGetLastError();
}

hipError_t gemm_launch(medusa_dtype dt, int epi, GemmBatch& bt, hipStream_t stream) {
    if (rowstream_eligible(dt, epi, bt.M, bt.K)) return launch_rowstream(epi, bt, stream);
    if (gemv_eligible(dt, epi, bt))
        return epi == EPI_TOPS ? launch_gemv_k<EPI_TOPS>(bt, stream) : launch_gemv_k<EPI_STORE>(bt, stream);
    return dt == MEDUSA_BF16 ? launch_epi<bf16_t>(epi, bt, stream) : launch_epi<float>(epi, bt, stream);
}

hipError_t topk_merge_launch(const MergeBatch& bt, hipStream_t stream) {
    for (int p = 0; p < bt.n_problems; ++p)
        if (bt.p[p].n_tiles > kMergeMaxTiles || bt.p[p].s > MEDUSA_MAX_TOPK) return hipErrorInvalidValue;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(bt.n_problems * bt.M), dim3(kThreads), 0, stream, bt);
    return hipGetLastError();
}

}  // namespace medusa
