// GEMMs of the decode step on gfx950: Y[m, n] = sum_k X[m, k] W[n, k] with W row-major
// [n, k] (the nn.Linear layout), fp32 accumulation and fused epilogues (bias/SiLU/residual
// store, per-tile top-s, per-tile argmax, typical-acceptance sums, fp32 slice sums).
//
// The weight matrix is the large operand, and a CU's vector memory path moves only so many
// bytes per second, so each kernel family is shaped by the bytes the busiest CU moves:
//   gemv_bf16_kernel          1-2 input rows (the heads at batch 1-2): whole rows of W per
//                             wave, 1 KiB per load instruction, dot products on the VALU;
//   gemm_rowstream_kernel     up to 64 rows (lm_head over the tree, heads from batch 3):
//                             8 rows x 128 B per load instruction through a wave-private
//                             LDS transpose into MFMA operands, input chunk shared in LDS;
//   gemm_cu_partial_kernel    the verifier's projections at 17-127 rows: one workgroup per
//                             CU, contraction slices summed by splitk_finalize_kernel;
//   gemm_tile_kernel          from 128 rows (argmax: above 64): 128 x 128, 128 x 256 or
//                             256 x 256 MFMA tiles, contraction slices for the projections;
//   gemm_splitk_rows_kernel   few rows with a store epilogue (the heads' feed-forward block
//                             from batch 3): the four waves split the contraction;
//   gemm_kernel, gemm_splitk_store_kernel, gemm_wave_partial_kernel   the shapes the above
//                             do not take (fp32, contractions or widths off their multiples).
// The MEDUSA_* macros below are compile-time tuning parameters; their defaults are the
// measured best on MI355X.
#include "common.hpp"
#include "internal.hpp"

#include <limits.h>

#include <algorithm>

namespace medusa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kLdsXBytes = 40960;     // X chunk budget (bytes of LDS)
constexpr int kSplitUnroll = 4;       // k-steps per load group in the split-contraction kernel
constexpr int kSplitRowsChunk = 64;   // contraction chunk of its row-contiguous bf16 form
#ifndef MEDUSA_SPLIT_ROWS
#define MEDUSA_SPLIT_ROWS 1
#endif
#ifndef MEDUSA_SPLIT_ROWS_PF
#define MEDUSA_SPLIT_ROWS_PF 3
#endif

// Streaming-kernel tiles: RT 16-row weight tiles per wave, UN k-steps per load group.
// Chosen by a sweep on MI355X at the 8B shape (RT in {1,2,4} x UN in {2,4,8}): the
// top-s (heads) launch is flat within a few percent across the sweep, the argmax
// (verify) launch prefers short groups.
template <typename T, int EPI> struct StreamCfg { static constexpr int RT = 2, UN = 4; };
template <> struct StreamCfg<bf16_t, EPI_TOPS> { static constexpr int RT = 2, UN = 8; };
template <> struct StreamCfg<bf16_t, EPI_ARGMAX> { static constexpr int RT = 2, UN = 2; };
template <typename T> struct StreamCfg<T, EPI_TYPICAL> : StreamCfg<T, EPI_ARGMAX> {};

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

#ifndef MEDUSA_SR_SWIZZLE
#define MEDUSA_SR_SWIZZLE 1
#endif
#ifndef MEDUSA_RS_SWIZZLE
#define MEDUSA_RS_SWIZZLE 1
#endif
#ifndef MEDUSA_TILE_SWIZZLE
#define MEDUSA_TILE_SWIZZLE 1
#endif
// LDS tiles of 64-element rows (128 B, 8 units of 16 B) with no padding: unit u of row r is
// stored at unit u ^ ((r >> 1) & 7).  A 16-lane group's 16-byte stores (two whole rows)
// then cover 64 distinct banks and its MFMA fragment reads (16 rows, one unit each) hit 16
// distinct 4-bank groups; a padded pitch of 72 made every pair of stored rows overlap.
__device__ __forceinline__ int sw64(int row, int col) {
    return row * 64 + ((((col >> 3) ^ (row >> 1)) & 7) << 3) + (col & 7);
}

// The same split for bf16 when every quarter of the contraction is whole 64-wide chunks:
// each wave streams its RT*16 weight rows over its quarter with row-contiguous loads (8
// rows x 128 B per instruction, the pattern that streams HBM fastest) into a wave-private,
// double-buffered LDS tile and reads the MFMA operands back from it, as the slice kernels
// do; input fragments come straight from the cache, rows past M are never read.  The four
// accumulators are summed in wave order through LDS, so the result is the same whichever
// wave finishes first.
template <int MT, int RT, int PF>
__global__ __launch_bounds__(kThreads) void gemm_splitk_rows_kernel(const GemmBatch bt) {
    constexpr int CH = kSplitRowsChunk;
    constexpr int KW = kWaves;
    constexpr int ROWS = 16 * RT;
    constexpr bool SWZ = MEDUSA_SR_SWIZZLE && CH == 64;
    constexpr int XP = SWZ ? CH : CH + 8;     // LDS pitch of a weight row (elements)
    auto at = [](int row, int c) __attribute__((always_inline)) { return SWZ ? sw64(row, c) : row * XP + c; };
    constexpr int LPR = CH / 8;               // lanes per weight row per load instruction
    constexpr int RPI = kWave / LPR;          // weight rows per load instruction
    constexpr int NI = ROWS / RPI;            // weight loads per lane per chunk
    constexpr int KS = CH / 32;               // MFMA steps per chunk
    static_assert(ROWS % RPI == 0, "rows per load");
    __shared__ __align__(16) bf16_t wt_all[KW][2][ROWS * XP];
    __shared__ floatx4 red[KW - 1][RT][MT][kWave];

    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    const int nblocks = bt.total_tiles * n_mb;
    const int bid = xcd_logical_block(blockIdx.x, nblocks);
    const int mb = bid % n_mb;
    const int t = bid / n_mb;
    const GemmProblem& P = bt.p[problem_of(bt, t)];
    const int tile = t - P.tile_begin;
    const int K = bt.K;
    const int N = P.N;
    const int kg = threadIdx.x >> 6;          // this wave's contraction quarter
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int n_wave = tile * ROWS;
    const int m0 = mb * MT * 16;
    const int n_ch = K / (CH * KW);           // chunks per quarter (the launch checks K)
    const int k_lo = kg * n_ch * CH;

    const bf16_t* W = static_cast<const bf16_t*>(P.W);
    const int half = lane / LPR;
    const int col = (lane % LPR) * 8;
    const u32x4* wsrc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int n = min(n_wave + RPI * i + half, N - 1);
        wsrc[i] = reinterpret_cast<const u32x4*>(W + (long long)n * K + k_lo + col);
    }
    const bf16_t* X = static_cast<const bf16_t*>(P.X);
    const bf16_t* xsrc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + mt * 16 + ln;
        long long r = m;
        bool ok = m < bt.M;
        if (ok && P.x_rows) {
            r = P.x_rows[m];
            ok = r >= 0 && r < bt.x_rows_bound;
        }
        xsrc[mt] = ok ? X + r * P.x_stride + k_lo + 8 * lg : nullptr;
    }

    floatx4 acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // rings: chunk j in slot j % PF; every load is issued on every path (chunks past the
    // quarter re-read its last one) so the compiler's wait counts stay exact
    u32x4 wr[PF][NI];
    Frag<bf16_t> xr[PF][MT][KS];
    // each tile walks its quarter from a chunk of its own (sums in that rotated order), so
    // concurrent tiles do not all read the same column offset of their 16 KiB-strided
    // rows at once: batched 70B heads 112.7 -> 109.7 us
    const int rot = n_ch > 0 ? (int)(((unsigned)tile * 37u) % (unsigned)n_ch) : 0;
    auto chunk_of = [&](int c) { int cr = min(c, n_ch - 1) + rot; return cr >= n_ch ? cr - n_ch : cr; };
    auto load_w = [&](int p, int c) {
        const int kc = chunk_of(c) * CH;
#pragma unroll
        for (int i = 0; i < NI; ++i) wr[p][i] = __builtin_nontemporal_load(wsrc[i] + kc / 8);
    };
    auto load_x = [&](int p, int c) {
        const int kc = chunk_of(c) * CH;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (xsrc[mt]) xr[p][mt][ks].load(xsrc[mt] + kc + 32 * ks);
                else xr[p][mt][ks].zero();
            }
    };
    bf16_t* wt = &wt_all[kg][0][0];
    auto store_w = [&](int p, int buf) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
            *reinterpret_cast<u32x4*>(&wt[buf * ROWS * XP + at(RPI * i + half, col)]) = wr[p][i];
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        load_w(p, p);
        load_x(p, p);
    }
    store_w(0, 0);
    load_w(0, PF);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int c0 = 0; c0 < n_ch; c0 += 2 * PF)
#pragma unroll
    for (int u = 0; u < 2 * PF; ++u) {
        const int c = c0 + u;
        if (c >= n_ch) break;
        const int ps = u % PF;                   // slot of chunk c
        const int pn = (u + 1) % PF;             // slot of chunk c + 1
        // weights of chunk c+1 into the other buffer, then refill their slot
        if (c + 1 < n_ch) store_w(pn, (u + 1) & 1);
        load_w(pn, c + 1 + PF);
        const bf16_t* wb = wt + (u & 1) * ROWS * XP;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            Frag<bf16_t> wf[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) wf[rt].load(wb + at(rt * 16 + ln, 32 * ks + 8 * lg));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) mma(acc[rt][mt], xr[ps][mt][ks], wf[rt]);
        }
        load_x(ps, c + PF);
        // wave-private buffer: a single-wave ordering point suffices
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
    for (int w = 0; w < KW - 1; ++w)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[rt][mt] += red[w][rt][mt][lane];
    store_epilogue<bf16_t, MT, RT>(P, bt, acc, m0, n_wave, ln, lg);
}

// EPI_TYPICAL after the argmax: the tile's softmax sums of every row and the logits of the
// tree candidates that fall in this wave's columns.  On entry red_v[0][row] holds the
// tile's maximum of each row (written by the argmax merge); red_v / red_i are then reused
// for the per-wave sums.  With x = (logit - tile max) / T: z = sum exp(x), s = sum exp(x) x.
template <int MT, int RT, int NWV>
__device__ __forceinline__ void typical_tile(const GemmProblem& P, const GemmBatch& bt,
                                             const floatx4 (&acc)[RT][MT], int m0, int Mb,
                                             int tile, int n_wave, int wave, int lane,
                                             float (&red_v)[NWV][MT * 16],
                                             int (&red_i)[NWV][MT * 16]) {
    const TypicalEpi& ty = bt.typ;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int N = P.N;
    constexpr float kLog2e = 1.4426950408889634f;
    __syncthreads();
    float tmax[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = mt * 16 + 4 * lg + r;
            tmax[mt][r] = row < Mb ? red_v[0][row] : 0.f;
        }
    __syncthreads();        // every lane has its maxima before the sums overwrite red_v
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float z = 0.f, sx = 0.f;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int n = n_wave + rt * 16 + ln;
                if (n < N) {
                    const float x = (acc[rt][mt][r] - tmax[mt][r]) * ty.inv_t;
                    const float e = __builtin_amdgcn_exp2f(x * kLog2e);
                    z += e;
                    sx += e * x;
                }
            }
            z = row_sum16(z);
            sx = row_sum16(sx);
            if (ln == 0) {
                red_v[wave][mt * 16 + 4 * lg + r] = z;
                red_i[wave][mt * 16 + 4 * lg + r] = __float_as_int(sx);
            }
        }
    __syncthreads();
    for (int m = threadIdx.x; m < Mb; m += NWV * kWave) {
        float z = red_v[0][m];
        float sx = __int_as_float(red_i[0][m]);
#pragma unroll
        for (int w = 1; w < NWV; ++w) {
            z += red_v[w][m];
            sx += __int_as_float(red_i[w][m]);
        }
        const long long o = (long long)(m0 + m) * P.n_tiles + tile;
        ty.part_z[o] = z;
        ty.part_s[o] = sx;
    }
    // Candidate logits: 64 candidates at a time, each lane loads one (parent row, token);
    // the few that fall in this wave's rows and columns are written by the lane holding them.
    const int NN = ty.n_nodes;
    const int b_lo = m0 / NN;
    const int b_hi = (m0 + Mb - 1) / NN;
    for (int b = b_lo; b <= b_hi; ++b) {
        for (int c0 = 1; c0 < NN; c0 += kWave) {
            const int c = c0 + lane;
            int pr = -1, tok = -1;
            if (c < NN) {
                pr = b * NN + ty.parent[c];
                tok = ty.node_tokens[(long long)b * NN + c];
            }
            const bool hit = c < NN && pr >= m0 && pr < m0 + Mb && tok >= n_wave &&
                             tok < n_wave + RT * 16;
            unsigned long long mask = __ballot(hit);
            while (mask) {
                const int src = __builtin_ctzll(mask);
                mask &= mask - 1;
                const int hp = __builtin_amdgcn_readlane(pr, src);
                const int ht = __builtin_amdgcn_readlane(tok, src);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n_wave + rt * 16 + ln == ht && m0 + mt * 16 + 4 * lg + r == hp)
                                ty.cand_logit[(long long)b * NN + c0 + src] = acc[rt][mt][r];
            }
        }
    }
}

// Shared epilogue of the MFMA kernels: optional fp32 logits, then the per-tile argmax or
// top-s of every input row.  acc[rt][mt][r] = Y[m0 + mt*16 + 4*lg + r][n_wave + rt*16 + ln];
// `smem` must hold Mb * NWG floats (top-s only) and may alias the kernel's X staging area.
template <int MT, int RT, int NWG, int EPI, int NWV = kWaves>
__device__ __forceinline__ void tile_epilogue(const GemmProblem& P, const GemmBatch& bt,
                                              const floatx4 (&acc)[RT][MT], int m0, int Mb,
                                              int tile, int n_wave, int wave, int lane,
                                              unsigned char* smem, float (&red_v)[NWV][MT * 16],
                                              int (&red_i)[NWV][MT * 16]) {
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

    if (EPI == EPI_ARGMAX || EPI == EPI_TYPICAL) {
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
        for (int m = threadIdx.x; m < Mb; m += NWV * kWave) {
            float bv = red_v[0][m];
            int bi = red_i[0][m];
#pragma unroll
            for (int w = 1; w < NWV; ++w)
                if (better(red_v[w][m], red_i[w][m], bv, bi)) { bv = red_v[w][m]; bi = red_i[w][m]; }
            const long long o = (long long)(m0 + m) * P.n_tiles + tile;
            P.part_val[o] = bv;
            P.part_idx[o] = bi;
            if (EPI == EPI_TYPICAL) red_v[0][m] = bv;     // this thread alone reads column m
        }
        if (EPI == EPI_TYPICAL)
            typical_tile<MT, RT, NWV>(P, bt, acc, m0, Mb, tile, n_wave, wave, lane, red_v, red_i);
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
        for (int m = wave; m < Mb; m += NWV) {
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

// Generic MFMA kernel (fp32, and bf16 shapes the specialised kernels do not take): each
// wave streams its RT*16 weight rows straight into MFMA operand registers (lane l reads 8
// elements of row l % 16 at contraction offset 8*(l/16), UN k-steps unrolled); the few X rows
// are staged through LDS in contraction chunks and shared by the four waves.
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
#define MEDUSA_RS_RTW 2
#endif
#ifndef MEDUSA_RS_PF
#define MEDUSA_RS_PF 1
#endif

constexpr int kRsChunk = MEDUSA_RS_CHUNK;   // contraction chunk per pass
#ifndef MEDUSA_RS_WAVES_TOPS
#define MEDUSA_RS_WAVES_TOPS 4
#endif
constexpr int kRsRtw = MEDUSA_RS_RTW;       // 16-row weight tiles per wave (top-s)
constexpr int kRsWavesTops = MEDUSA_RS_WAVES_TOPS;
constexpr int kRsPf = MEDUSA_RS_PF;         // chunks in flight ahead of the one multiplied
// The top-s path (heads from batch 3) streams 256-wide chunks: at batch 8 of the 70B shape
// heads_vocab took 391.7 us against 413.8 with 64-wide chunks (128: 412.0; 512: 420.3),
// 0.96 of the read probe.  Each chunk costs two block barriers and an LDS round trip, which
// a wider chunk pays less often per weight byte.  Contractions that 256 does not divide
// keep the 64-wide chunk.
#ifndef MEDUSA_RS_CHUNK_TOPS
#define MEDUSA_RS_CHUNK_TOPS 256
#endif
constexpr int kRsChunkTops = MEDUSA_RS_CHUNK_TOPS;
constexpr int kPartialChunk = 64;           // contraction chunk of the slice kernels
constexpr int kWavePartialRows = 64;        // weight rows per single-wave slice tile
#ifndef MEDUSA_RS_WAVES_ARGMAX
#define MEDUSA_RS_WAVES_ARGMAX 8
#endif
#ifndef MEDUSA_RS_RTW_ARGMAX
#define MEDUSA_RS_RTW_ARGMAX 2
#endif
// Argmax path (lm_head over the tree nodes): 8 waves of 32 rows per workgroup, two
// workgroups per CU.  Measured at the 8B shape (64 nodes): 4 x 64 rows 161 us, 8 x 32 158,
// 8 x 64 181 (one workgroup per CU; its eight-wave barrier gates every chunk), 16 x 32 176.
constexpr int kRsWavesArgmax = MEDUSA_RS_WAVES_ARGMAX;
constexpr int kRsRtwArgmax = MEDUSA_RS_RTW_ARGMAX;
// A small vocabulary leaves CUs idle with 256-row tiles (32000 rows are 125 tiles for 256
// CUs): below 65536 rows the argmax and typical paths at up to 64 verified rows take
// 4 waves of 16 rows, 64-row tiles.  Measured at the 7B shape (vocabulary 32000, 64
// nodes): 256-row tiles 107.8 us, 128 (4 x 32) 82.4, 128 (8 x 16) 82.9, 64 (2 x 32) 80.1,
// 64 (4 x 16) 75.9.
#ifndef MEDUSA_RS_SMALL_VOCAB
#define MEDUSA_RS_SMALL_VOCAB 65536
#endif
#ifndef MEDUSA_RS_WAVES_SMALLV
#define MEDUSA_RS_WAVES_SMALLV 4
#endif
#ifndef MEDUSA_RS_RTW_SMALLV
#define MEDUSA_RS_RTW_SMALLV 1
#endif
// Small vocabulary: 256-wide contraction chunks, one in flight (7B verify 55.8 -> 53.7 us
// against 64-wide chunks two in flight, 73.5 us with one): a quarter of the chunks, so a
// quarter of the block barriers and LDS round trips per weight byte.  Contractions that
// 256 does not divide keep the 64-wide chunks, two in flight.
#ifndef MEDUSA_RS_PF_SMALLV
#define MEDUSA_RS_PF_SMALLV 1
#endif
#ifndef MEDUSA_RS_CHUNK_SMALLV
#define MEDUSA_RS_CHUNK_SMALLV 256
#endif
constexpr int kRsWavesSmallVocab = MEDUSA_RS_WAVES_SMALLV;
constexpr int kRsRtwSmallVocab = MEDUSA_RS_RTW_SMALLV;
bool rs_small_vocab(int M, int N) { return M <= 64 && N < MEDUSA_RS_SMALL_VOCAB; }

template <int MT, int EPI, int RTW, int PF, int CH, int NWV>
__global__ __launch_bounds__(NWV * kWave) void gemm_rowstream_kernel(const GemmBatch bt) {
    constexpr int RT = RTW;
    constexpr int ROWS = 16 * RT;             // weight rows per wave
    constexpr int NWG = NWV * ROWS;
    constexpr int NTH = NWV * kWave;
    constexpr bool SWZ = MEDUSA_RS_SWIZZLE && CH == 64;
    constexpr int XP = SWZ ? CH : CH + 8;     // LDS pitch of X rows and W tiles (elements)
    auto at = [](int row, int c) __attribute__((always_inline)) { return SWZ ? sw64(row, c) : row * XP + c; };
    constexpr int LPR = CH / 8;               // lanes per row in one load instruction
    constexpr int RPI = kWave / LPR;          // rows per load instruction
    constexpr int NI = ROWS / RPI;            // 16-byte loads per lane per chunk
    constexpr int VPR = CH / 8;               // 16-byte vectors per X row chunk
    constexpr int XV = (MT * 16 * VPR + NTH - 1) / NTH;   // ... per thread
    // X rows past the tile land in a spare slot at the end (every thread stores); the
    // layout is rowstream_lds()'s
    extern __shared__ __align__(16) unsigned char rs_lds[];
    bf16_t* xs = reinterpret_cast<bf16_t*>(rs_lds);                          // [MT*16*XP + 8]
    auto& wt = *reinterpret_cast<bf16_t (*)[NWV][ROWS * XP]>(xs + MT * 16 * XP + 8);
    auto& red_v = *reinterpret_cast<float (*)[NWV][MT * 16]>(&wt[NWV][0]);
    auto& red_i = *reinterpret_cast<int (*)[NWV][MT * 16]>(&red_v[NWV][0]);

    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    const int nblocks = bt.total_tiles * n_mb;
    const int bid = xcd_logical_block(blockIdx.x, nblocks);
    const int mb = bid % n_mb;
    const int t = bid / n_mb;
    const GemmProblem& P = bt.p[problem_of(bt, t)];
    const int tile = t - P.tile_begin;
    const int K = bt.K;
    const int N = P.N;
    const int k_lo = 0;
    const int k_hi = K;
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
    const bf16_t* X = static_cast<const bf16_t*>(P.X);
    bf16_t* wtile = wt[wave];

    floatx4 acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // X vectors of this thread: rows without a source (past M, or an out-of-range gather
    // index) read row 0 and are replaced by zeros before the LDS store
    const bf16_t* xrow_ptr[XV];
    bool xok[XV];
    int xdst[XV];
#pragma unroll
    for (int j = 0; j < XV; ++j) {
        const int idx = threadIdx.x + j * NTH;
        const int m = idx / VPR;
        const int c = idx - m * VPR;
        xdst[j] = m < MT * 16 ? at(m, c * 8) : MT * 16 * XP;
        long long r = 0;
        bool ok = m < Mb;
        if (ok) {
            r = m0 + m;
            if (P.x_rows) {
                r = P.x_rows[m0 + m];
                ok = r >= 0 && r < bt.x_rows_bound;
                if (!ok) r = 0;
            }
        }
        xok[j] = ok;
        xrow_ptr[j] = X + r * P.x_stride + c * 8;
    }

    // Ring of PF chunks in registers; chunk c of the slice lives in slot c % PF.  Every
    // load is issued on every path (refills past the slice re-read its last chunk) so the
    // compiler's wait counts stay exact: storing slot p waits only for slot p's loads.
    const int n_ch = (k_hi - k_lo) / CH;
    // With 64-wide chunks every tile starts its walk over the contraction at its own
    // chunk (the sums are taken in that rotated order).  Tiles that all read the same
    // column offset of their 8 KiB-strided rows at the same moment otherwise crowd the
    // same memory channels: 8B-shape verification 168.6 -> 160.5 us.
    const int rot = CH == 64 && n_ch > 0 ? (int)(((unsigned)tile * 37u) % (unsigned)n_ch) : 0;
    u32x4 wr[PF][NI];
    u32x4 xr[PF][XV];
    auto load = [&](int p, int c) {
        int cr = min(c, n_ch - 1) + rot;
        if (cr >= n_ch) cr -= n_ch;
        const int kc = k_lo + cr * CH;
#pragma unroll
        for (int i = 0; i < NI; ++i) wr[p][i] = __builtin_nontemporal_load(wsrc[i] + kc / 8);
#pragma unroll
        for (int j = 0; j < XV; ++j) xr[p][j] = *reinterpret_cast<const u32x4*>(xrow_ptr[j] + kc);
    };
    if (n_ch > 0) {
#pragma unroll
        for (int p = 0; p < PF; ++p) load(p, p);
    }
    for (int c0 = 0; c0 < n_ch; c0 += PF)
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        const int c = c0 + p;
        if (c >= n_ch) break;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < XV; ++j) {
            const u32x4 v = xok[j] ? xr[p][j] : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(xs + xdst[j]) = v;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
            *reinterpret_cast<u32x4*>(wtile + at(RPI * i + half, col)) = wr[p][i];
        __syncthreads();
        load(p, c + PF);
#pragma unroll
        for (int ks = 0; ks < CH; ks += 32) {
            Frag<bf16_t> wf[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) wf[rt].load(wtile + at(rt * 16 + ln, ks + 8 * lg));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                Frag<bf16_t> xf;       // rows past Mb hold zeros
                xf.load(xs + at(mt * 16 + ln, ks + 8 * lg));
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) mma(acc[rt][mt], xf, wf[rt]);
            }
        }
    }
    // the top-s epilogue needs Mb * NWG floats of scratch: the W tiles are free by now
    static_assert(EPI != EPI_TOPS || sizeof(bf16_t) * NWV * ROWS * XP >= 16 * NWG * sizeof(float),
                  "top-s scratch");
    __syncthreads();
    tile_epilogue<MT, RT, NWG, EPI, NWV>(P, bt, acc, m0, Mb, tile, n_wave, wave, lane,
                                         reinterpret_cast<unsigned char*>(&wt[0][0]), red_v, red_i);
}

// Single-wave contraction slices for the verifier's projections (many input rows, small
// weights).  One wave per workgroup owns 16*RT weight rows, MT*16 input rows and one
// contraction slice, so no step waits for another wave: the weight chunk is transposed
// through a wave-private, double-buffered LDS tile (the store of chunk c+1 overlaps the
// products of chunk c; one single-wave barrier per chunk) and the input rows are loaded
// straight from the cache in the MFMA operand layout (16 input rows x 8 contraction
// elements per lane and step).  Weight and input chunks run PF chunks ahead in registers.
// The slice sums go to part_val like the row-streaming kernel's, and the same finalize
// pass sums them.
template <int MT, int RT, int PF, int CH>
__global__ __launch_bounds__(kWave) void gemm_wave_partial_kernel(const GemmBatch bt) {
    constexpr int ROWS = 16 * RT;
    constexpr int XP = CH + 8;                // LDS pitch of a weight row (elements)
    constexpr int LPR = CH / 8;               // lanes per weight row per load instruction
    constexpr int RPI = kWave / LPR;          // weight rows per load instruction
    constexpr int NI = ROWS / RPI;            // weight loads per lane per chunk
    constexpr int KS = CH / 32;               // MFMA steps per chunk
    constexpr int XL = MT * KS;               // input loads per lane per chunk
    static_assert(ROWS % RPI == 0, "rows per load");
    __shared__ __align__(16) bf16_t wt[2][ROWS * XP];

    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    const int nks = bt.ksplit;
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
    const int chunks = K / CH;
    const int per = (chunks + nks - 1) / nks;
    const int c_lo = min(chunks, ksl * per);
    const int n_ch = min(chunks, (ksl + 1) * per) - c_lo;
    const int k_lo = c_lo * CH;
    const int lane = threadIdx.x;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int n0 = tile * ROWS;
    const int m0 = mb * MT * 16;

    const bf16_t* W = static_cast<const bf16_t*>(P.W);
    const int half = lane / LPR;
    const int col = (lane % LPR) * 8;
    const u32x4* wsrc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int n = min(n0 + RPI * i + half, N - 1);
        wsrc[i] = reinterpret_cast<const u32x4*>(W + (long long)n * K + k_lo + col);
    }
    // input row of m-tile mt for this lane: rows without a source read row 0, zeroed later
    const bf16_t* X = static_cast<const bf16_t*>(P.X);
    const bf16_t* xsrc[MT];
    bool xok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + mt * 16 + ln;
        long long r = 0;
        bool ok = m < bt.M;
        if (ok) {
            r = m;
            if (P.x_rows) {
                r = P.x_rows[m];
                ok = r >= 0 && r < bt.x_rows_bound;
                if (!ok) r = 0;
            }
        }
        xok[mt] = ok;
        xsrc[mt] = X + r * P.x_stride + k_lo + 8 * lg;
    }

    floatx4 acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // rings: chunk j in slot j % PF; every load is issued on every path (chunks past the
    // slice re-read its last one) so the compiler's wait counts stay exact
    u32x4 wr[PF][NI];
    u32x4 xr[PF][XL];
    auto load_w = [&](int p, int c) {
        const int kc = min(c, n_ch - 1) * CH;
#pragma unroll
        for (int i = 0; i < NI; ++i) wr[p][i] = __builtin_nontemporal_load(wsrc[i] + kc / 8);
    };
    auto load_x = [&](int p, int c) {
        const int kc = min(c, n_ch - 1) * CH;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                xr[p][mt * KS + ks] = *reinterpret_cast<const u32x4*>(xsrc[mt] + kc + 32 * ks);
    };
    auto store_w = [&](int p, int buf) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
            *reinterpret_cast<u32x4*>(&wt[buf][(RPI * i + half) * XP + col]) = wr[p][i];
    };
    if (n_ch > 0) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            load_w(p, p);
            load_x(p, p);
        }
        store_w(0, 0);
        load_w(0, PF);
        __syncthreads();
        for (int c0 = 0; c0 < n_ch; c0 += 2 * PF)
#pragma unroll
        for (int u = 0; u < 2 * PF; ++u) {
            const int c = c0 + u;
            if (c >= n_ch) break;
            const int ps = u % PF;               // slot of chunk c
            const int pn = (u + 1) % PF;         // slot of chunk c + 1
            // weights of chunk c+1 into the other buffer, then refill their slot
            if (c + 1 < n_ch) store_w(pn, (u + 1) & 1);
            load_w(pn, c + 1 + PF);
            const bf16_t* wb = wt[u & 1];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Frag<bf16_t> wf[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) wf[rt].load(wb + (rt * 16 + ln) * XP + 32 * ks + 8 * lg);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    Frag<bf16_t> xf;
                    xf.v = xok[mt] ? xr[ps][mt * KS + ks] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) mma(acc[rt][mt], xf, wf[rt]);
                }
            }
            load_x(ps, c + PF);
            __syncthreads();
        }
    }
    float* part = P.part_val + (long long)ksl * bt.M * N;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int n = n0 + rt * 16 + ln;
        if (n >= N) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + mt * 16 + 4 * lg + r;
                if (m < bt.M) part[(long long)m * N + n] = acc[rt][mt][r];
            }
    }
}

// One workgroup per compute unit for the verifier's projections.  Every CU's vector memory
// path moves only so many bytes per second (about 27 GB/s per CU at full HBM rate), so a
// small, latency-exposed GEMM streams fastest when each of the 256 CUs carries the same
// weight bytes and little else.  A workgroup owns NW*32 weight rows (a wave per 32 rows;
// the rows may run across the batch's problems, whose sizes are multiples of 32) and one
// contraction slice: it stages the slice of the (gathered) input rows in LDS once, then
// every wave streams its rows like gemm_wave_partial_kernel (register ring, private
// double-buffered transpose) with the input operands read from the shared slice.
constexpr int kCuRt = 2;                     // 16-row tiles per wave
constexpr int kCuChunk = 64;
constexpr int kCuXv = 16;                    // staged input vectors per thread per batch

template <int NW, int PF>
__global__ __launch_bounds__(NW * kWave) void gemm_cu_partial_kernel(const GemmBatch bt, int rows_total) {
    constexpr int MT = 4;
    constexpr int RT = kCuRt;
    constexpr int CH = kCuChunk;
    constexpr int ROWS = 16 * RT;
    constexpr int R = NW * ROWS;
    constexpr int XP = CH + 8;
    constexpr int LPR = CH / 8;
    constexpr int RPI = kWave / LPR;
    constexpr int NI = ROWS / RPI;
    constexpr int KS = CH / 32;
    constexpr int NT = NW * kWave;
    extern __shared__ __align__(16) unsigned char dyn_smem[];

    const int nks = bt.ksplit;
    const int n_rt = (rows_total + R - 1) / R;
    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    const int nblocks = n_rt * n_mb * nks;
    int bid = xcd_logical_block(blockIdx.x, nblocks);
    const int mb = bid % n_mb;
    bid /= n_mb;
    const int ksl = bid % nks;
    const int rtile = bid / nks;
    const int K = bt.K;
    const int chunks = K / CH;
    const int per = (chunks + nks - 1) / nks;
    const int c_lo = min(chunks, ksl * per);
    const int n_ch = min(chunks, (ksl + 1) * per) - c_lo;
    const int k_lo = c_lo * CH;
    const int XPK = per * CH + 8;                            // LDS pitch of the input slice
    bf16_t* xs = reinterpret_cast<bf16_t*>(dyn_smem);        // [MT*16][XPK]
    bf16_t* wt_all = xs + MT * 16 * XPK;                     // [NW][2][ROWS*XP]
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int m0 = mb * MT * 16;

    // this wave's rows in the concatenation of the problems
    const int g0 = rtile * R + wave * ROWS;
    int p = 0, rb = 0;
    while (p < bt.n_problems - 1 && g0 >= rb + bt.p[p].N) rb += bt.p[p++].N;
    const GemmProblem& P = bt.p[p];
    const bool active = g0 < rows_total;
    const int n0 = active ? g0 - rb : 0;
    const int my_ch = active ? n_ch : 0;        // waves past the last row stream nothing
    const int N = P.N;

    const bf16_t* W = static_cast<const bf16_t*>(P.W);
    const int half = lane / LPR;
    const int col = (lane % LPR) * 8;
    const u32x4* wsrc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int n = min(n0 + RPI * i + half, N - 1);
        wsrc[i] = reinterpret_cast<const u32x4*>(W + (long long)n * K + k_lo + col);
    }
    u32x4 wr[PF][NI];
    auto load_w = [&](int q, int c) {
        const int kc = min(c, my_ch - 1) * CH;
#pragma unroll
        for (int i = 0; i < NI; ++i) wr[q][i] = __builtin_nontemporal_load(wsrc[i] + kc / 8);
    };
    bf16_t* wt = wt_all + wave * 2 * ROWS * XP;
    auto store_w = [&](int q, int buf) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
            *reinterpret_cast<u32x4*>(&wt[buf * ROWS * XP + (RPI * i + half) * XP + col]) = wr[q][i];
    };
    if (my_ch > 0) {
#pragma unroll
        for (int q = 0; q < PF; ++q) load_w(q, q);
    }

    // input slice: rows m0.. of the (shared) input, columns k_lo .. k_lo + n_ch*CH; rows
    // without a source are zero.  The gather indices are resolved once into LDS, then every
    // row load is issued unconditionally (kCuXv per thread before their stores), so the
    // loads overlap instead of waiting one by one.
    {
        __shared__ int xrow[MT * 16];
        const GemmProblem& P0 = bt.p[0];
        if (threadIdx.x < MT * 16) {
            const int m = m0 + threadIdx.x;
            int r = -1;
            if (m < bt.M) {
                r = m;
                if (P0.x_rows) {                 // gathered rows: out-of-range indices read zeros
                    r = P0.x_rows[m];
                    if (r < 0 || r >= bt.x_rows_bound) r = -1;
                }
            }
            xrow[threadIdx.x] = r;
        }
        __syncthreads();
        const bf16_t* X = static_cast<const bf16_t*>(P0.X) + k_lo;
        const int vpr = n_ch * CH / 8;
        const int total = MT * 16 * vpr;
        for (int base = 0; base < total; base += NT * kCuXv) {
            u32x4 v[kCuXv];
            int dst[kCuXv];
#pragma unroll
            for (int j = 0; j < kCuXv; ++j) {
                const int idx = min(base + j * NT + (int)threadIdx.x, total - 1);
                const int m = idx / vpr;
                const int c = idx - m * vpr;
                const int r = xrow[m];
                dst[j] = base + j * NT + (int)threadIdx.x < total ? (r >= 0 ? m * XPK + c * 8 : -(m * XPK + c * 8) - 1) : INT_MIN;
                v[j] = *reinterpret_cast<const u32x4*>(X + (long long)max(r, 0) * P0.x_stride + c * 8);
            }
#pragma unroll
            for (int j = 0; j < kCuXv; ++j) {
                if (dst[j] == INT_MIN) continue;
                const bool ok = dst[j] >= 0;
                *reinterpret_cast<u32x4*>(xs + (ok ? dst[j] : -dst[j] - 1)) = ok ? v[j] : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    floatx4 acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    if (my_ch > 0) {
        store_w(0, 0);
        load_w(0, PF);
    }
    __syncthreads();
    if (my_ch > 0) {
        for (int c0 = 0; c0 < my_ch; c0 += 2 * PF)
#pragma unroll
        for (int u = 0; u < 2 * PF; ++u) {
            const int c = c0 + u;
            if (c >= my_ch) break;
            const int pn = (u + 1) % PF;
            if (c + 1 < my_ch) store_w(pn, (u + 1) & 1);
            load_w(pn, c + 1 + PF);
            const bf16_t* wb = wt + (u & 1) * ROWS * XP;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Frag<bf16_t> wf[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) wf[rt].load(wb + (rt * 16 + ln) * XP + 32 * ks + 8 * lg);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    Frag<bf16_t> xf;
                    xf.load(xs + (mt * 16 + ln) * XPK + c * CH + 32 * ks + 8 * lg);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) mma(acc[rt][mt], xf, wf[rt]);
                }
            }
            // wave-private buffer: a single-wave ordering point suffices
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
    if (!active) return;
    float* part = P.part_val + (long long)ksl * bt.M * N;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int n = n0 + rt * 16 + ln;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + mt * 16 + 4 * lg + r;
                if (m < bt.M) part[(long long)m * N + n] = acc[rt][mt][r];
            }
    }
}

// Four consecutive elements as fp32, through one 8-byte (bf16) or 16-byte (fp32) access.
template <typename T> __device__ __forceinline__ void load4(const T* p, float (&v)[4]);
template <> __device__ __forceinline__ void load4<float>(const float* p, float (&v)[4]) {
    const floatx4 q = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = q[j];
}
template <> __device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float (&v)[4]) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xFFFF0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xFFFF0000u);
}
template <typename T> __device__ __forceinline__ void store4(T* p, const float (&v)[4]);
template <> __device__ __forceinline__ void store4<float>(float* p, const float (&v)[4]) {
    *reinterpret_cast<floatx4*>(p) = floatx4{v[0], v[1], v[2], v[3]};
}
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float (&v)[4]) {
    uint2 q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = q;
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
    if (N % 4 == 0) {
        // one 16-byte load per slice, all slices in flight before the (ordered) sum
        constexpr int kMaxSlices = 16;
        floatx4 sv[kMaxSlices];
        const floatx4* base = reinterpret_cast<const floatx4*>(P.part_val + (long long)m * N + n0);
        const long long stride = (long long)bt.M * N / 4;
#pragma unroll
        for (int ks = 0; ks < kMaxSlices; ++ks)
            if (ks < bt.ksplit) sv[ks] = base[ks * stride];
#pragma unroll
        for (int ks = 0; ks < kMaxSlices; ++ks)
            if (ks < bt.ksplit)
#pragma unroll
                for (int j = 0; j < 4; ++j) y[j] += sv[ks][j];
        for (int ks = kMaxSlices; ks < bt.ksplit; ++ks)
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] += base[ks * stride][j];
    } else {
        for (int ks = 0; ks < bt.ksplit; ++ks) {
            const float* part = P.part_val + ((long long)ks * bt.M + m) * N;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n0 + j < N) y[j] += part[n0 + j];
        }
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
    T* dst = out + (long long)m * P.ldo + n0;
    const T* bsrc = bias ? bias + n0 : nullptr;
    const T* rsrc = rok ? res + rr * P.res_stride + n0 : nullptr;
    // four whole, aligned elements (every thread of a launch agrees): one vector access each
    // for the bias, the residual and the output instead of four scalar ones
    constexpr uintptr_t kVec = 4 * sizeof(T) - 1;
    const bool vec = n0 + 4 <= N && ((uintptr_t)dst & kVec) == 0 &&
                     (!bsrc || ((uintptr_t)bsrc & kVec) == 0) && (!rsrc || ((uintptr_t)rsrc & kVec) == 0);
    if (vec) {
        float bv[4] = {0.f, 0.f, 0.f, 0.f}, rv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bsrc) load4<T>(bsrc, bv);
        if (rsrc) load4<T>(rsrc, rv);
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = y[j] + bv[j];
            if (P.silu) v[j] = silu(v[j]);
            if (rsrc) v[j] += rv[j];
        }
        store4<T>(dst, v);
        return;
    }
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


// Tiled MFMA GEMM for many input rows: the verifier's projections from 128 verified rows
// (256 x 256 tiles in contraction slices, or 128 x 128 tiles with the store epilogue when
// one slice is best; the contraction is compute-heavy there: 512 rows at the 70B shape
// are 512 flops per weight byte) and lm_head over more than 64 verified rows (argmax
// epilogue).  A workgroup of WM x WN waves owns a (16*WM*MTW) x (16*WN*RTW) tile of
// Y = X W^T, each wave a (16*MTW) x (16*RTW) block, and walks the contraction in 64-wide
// chunks: the chunk's X and W rows are loaded into registers one chunk ahead (8 lanes x
// 16 B per row per instruction; gathered X rows without a source read row 0 and are
// zeroed), stored into LDS, and read back in the MFMA operand layout.  The workgroups
// sharing a W tile are neighbours in the XCD-aware numbering, so the tile leaves HBM once.
// With DB the LDS holds two chunks: chunk c+1 is stored while chunk c is multiplied, and
// one block barrier per chunk orders them.  EPI_PARTIAL splits the contraction into
// bt.ksplit slices and writes each slice's fp32 sums to part_val[slice][m][n] for the
// finalize pass.  The LDS layout is tile_lds()'s.
template <int WM, int WN, int MTW, int RTW, bool DB = false>
constexpr size_t tile_lds() {
    return (size_t)(16 * WM * MTW + 16 * WN * RTW) * (MEDUSA_TILE_SWIZZLE ? 64 : 64 + 8) * 2 * (DB ? 2 : 1) +
           (size_t)WN * 16 * WM * MTW * 8;
}

template <int WM, int WN, int MTW, int RTW, int EPI, bool DB = false>
__global__ __launch_bounds__(WM * WN * kWave) void gemm_tile_kernel(const GemmBatch bt) {
    constexpr int NT = WM * WN * kWave;
    constexpr int TM = 16 * WM * MTW;           // input rows per tile
    constexpr int TN = 16 * WN * RTW;           // weight rows per tile
    constexpr int CH = 64;
    constexpr int XP = MEDUSA_TILE_SWIZZLE ? CH : CH + 8;    // see sw64()
    auto sw = [](int row, int col) __attribute__((always_inline)) {   // element offset in an LDS tile
        return MEDUSA_TILE_SWIZZLE ? sw64(row, col) : row * (CH + 8) + col;
    };
    constexpr int LPR = CH / 8;                 // lanes per row per load instruction
    constexpr int RPI = NT / LPR;               // rows per workgroup load instruction
    constexpr int XL = TM / RPI;                // X loads per thread per chunk
    constexpr int WL = TN / RPI;                // W loads per thread per chunk
    static_assert(XL >= 1 && WL >= 1 && XL * RPI == TM && WL * RPI == TN, "tile rows");
    constexpr int STAGE = (TM + TN) * XP;       // elements of one chunk's X and W rows
    extern __shared__ __align__(16) unsigned char tile_smem[];
    bf16_t* const lds0 = reinterpret_cast<bf16_t*>(tile_smem);   // [DB?2:1][TM+TN][XP]
    auto& red_v = *reinterpret_cast<float (*)[WN][TM]>(lds0 + STAGE * (DB ? 2 : 1));
    auto& red_i = *reinterpret_cast<int (*)[WN][TM]>(&red_v[WN][0]);

    const int n_mb = (bt.M + TM - 1) / TM;
    const int nks = EPI == EPI_PARTIAL ? bt.ksplit : 1;
    const int nblocks = bt.total_tiles * n_mb * nks;
    int bid = xcd_logical_block(blockIdx.x, nblocks);
    const int mb = bid % n_mb;
    bid /= n_mb;
    const int ksl = bid % nks;                  // contraction slice (EPI_PARTIAL)
    const int t = bid / nks;
    const GemmProblem& P = bt.p[problem_of(bt, t)];
    const int tile = t - P.tile_begin;
    const int K = bt.K;
    const int N = P.N;
    const int m0 = mb * TM;
    const int n0 = tile * TN;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int wmi = wave % WM;                  // the wave's block within the tile
    const int wni = wave / WM;
    const int wm = wmi * 16 * MTW;
    const int wn = wni * 16 * RTW;

    const int lrow = threadIdx.x / LPR;         // row of this thread's loads (plus RPI * i)
    const int lcol = (threadIdx.x % LPR) * 8;
    const bf16_t* X = static_cast<const bf16_t*>(P.X);
    const bf16_t* W = static_cast<const bf16_t*>(P.W);
    const bf16_t* xsrc[XL];
    bool xok[XL];
#pragma unroll
    for (int i = 0; i < XL; ++i) {
        const int m = m0 + lrow + RPI * i;
        long long r = 0;
        bool ok = m < bt.M;
        if (ok) {
            r = m;
            if (P.x_rows) {
                r = P.x_rows[m];
                ok = r >= 0 && r < bt.x_rows_bound;
                if (!ok) r = 0;
            }
        }
        xok[i] = ok;
        xsrc[i] = X + r * P.x_stride + lcol;
    }
    const bf16_t* wsrc[WL];
#pragma unroll
    for (int i = 0; i < WL; ++i)
        wsrc[i] = W + (long long)min(n0 + lrow + RPI * i, N - 1) * K + lcol;

    // this workgroup's chunks: all of them, or its slice's
    const int chunks = K / CH;
    const int per = (chunks + nks - 1) / nks;
    const int c_lo = min(chunks, ksl * per);
    const int n_ch = min(chunks, (ksl + 1) * per) - c_lo;
    u32x4 xr[XL], wr[WL];
    // Verification tiles start their walk over the contraction at a chunk of their own
    // (both row blocks of a W tile at the same one, so the tile still leaves HBM once),
    // which spreads the reads of concurrent tiles over the memory channels, when all of X
    // fits an XCD's L2 comfortably (at most 2 MiB): dense tree 223.8 -> 214.4 us.  With a
    // larger X (batched 70B, 8 MiB) the rotated walks no longer share X in L2 and lose.
    const int rot = EPI == EPI_ARGMAX && n_ch > 0 && (long long)bt.M * K * 2 <= (2ll << 20)
                        ? (int)(((unsigned)t * 37u) % (unsigned)n_ch) : 0;
    auto load = [&](int c) {
        int cr = min(c, n_ch - 1) + rot;
        if (cr >= n_ch) cr -= n_ch;
        const int kc = (c_lo + cr) * CH;
#pragma unroll
        for (int i = 0; i < XL; ++i) xr[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + kc);
#pragma unroll
        for (int i = 0; i < WL; ++i)
            wr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc[i] + kc));
    };
    auto stash = [&](bf16_t* st) {              // the loaded chunk into one LDS stage
        bf16_t* xs = st;
        bf16_t* ws = st + TM * XP;
#pragma unroll
        for (int i = 0; i < XL; ++i)
            *reinterpret_cast<u32x4*>(xs + sw(lrow + RPI * i, lcol)) = xok[i] ? xr[i] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < WL; ++i)
            *reinterpret_cast<u32x4*>(ws + sw(lrow + RPI * i, lcol)) = wr[i];
    };

    floatx4 acc[RTW][MTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) acc[rt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto multiply = [&](const bf16_t* st) {     // acc += the chunk in one LDS stage
        const bf16_t* xs = st;
        const bf16_t* ws = st + TM * XP;
        // a wave raises its issue priority while it multiplies, so that the waves sharing
        // its SIMD and still staging a chunk yield the issue slots to the matrix work
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < CH; ks += 32) {
            Frag<bf16_t> wf[RTW];
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) wf[rt].load(ws + sw(wn + rt * 16 + ln, ks + 8 * lg));
            // the next X fragment is read while the current one's MFMAs run
            Frag<bf16_t> xf[2];
            xf[0].load(xs + sw(wm + ln, ks + 8 * lg));
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) {
                if (mt + 1 < MTW) xf[(mt + 1) & 1].load(xs + sw(wm + (mt + 1) * 16 + ln, ks + 8 * lg));
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt) mma(acc[rt][mt], xf[mt & 1], wf[rt]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    if (n_ch > 0) load(0);
    if (DB) {
        // stage c & 1 holds chunk c.  Storing chunk c+1 into the other stage is safe: its
        // last readers multiplied chunk c-1 before the barrier that ended that iteration.
        if (n_ch > 0) {
            stash(lds0);
            load(1);
        }
        __syncthreads();
        for (int c = 0; c < n_ch; ++c) {
            multiply(lds0 + (c & 1) * STAGE);
            if (c + 1 < n_ch) {
                stash(lds0 + ((c + 1) & 1) * STAGE);
                load(c + 2);
            }
            __syncthreads();
        }
    } else {
        for (int c = 0; c < n_ch; ++c) {
            __syncthreads();
            stash(lds0);
            __syncthreads();
            load(c + 1);
            multiply(lds0);
        }
    }
    if (EPI == EPI_STORE) {
        store_epilogue<bf16_t, MTW, RTW>(P, bt, acc, m0 + wm, n0 + wn, ln, lg);
        return;
    }
    if (EPI == EPI_PARTIAL) {
        float* part = P.part_val + (long long)ksl * bt.M * N;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            const int n = n0 + wn + rt * 16 + ln;
            if (n >= N) continue;
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + wm + mt * 16 + 4 * lg + r;
                    if (m < bt.M) part[(long long)m * N + n] = acc[rt][mt][r];
                }
        }
        return;
    }
    // EPI_ARGMAX: optional fp32 logits, then each wave's best (value, id) per row over its
    // columns, and the WN waves that share the rows combine in a fixed order; one partial
    // per (row, tile)
    if (P.logits) {
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            const int n = n0 + wn + rt * 16 + ln;
            if (n >= N) continue;
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + wm + mt * 16 + 4 * lg + r;
                    if (m < bt.M) P.logits[(long long)m * P.logits_ld + n] = acc[rt][mt][r];
                }
        }
    }
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float bv = -INFINITY;
            int bi = INT_MAX;
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) {
                const int n = n0 + wn + rt * 16 + ln;
                const float v = n < N ? acc[rt][mt][r] : -INFINITY;
                const int id = n < N ? n : INT_MAX;
                if (better(v, id, bv, bi)) { bv = v; bi = id; }
            }
            row_best(bv, bi);
            if (ln == 0) {
                red_v[wni][wm + mt * 16 + 4 * lg + r] = bv;
                red_i[wni][wm + mt * 16 + 4 * lg + r] = bi;
            }
        }
    __syncthreads();
    const int Mb = min(bt.M - m0, TM);
    for (int m = threadIdx.x; m < Mb; m += NT) {
        float bv = red_v[0][m];
        int bi = red_i[0][m];
#pragma unroll
        for (int w = 1; w < WN; ++w)
            if (better(red_v[w][m], red_i[w][m], bv, bi)) { bv = red_v[w][m]; bi = red_i[w][m]; }
        const long long o = (long long)(m0 + m) * P.n_tiles + tile;
        P.part_val[o] = bv;
        P.part_idx[o] = bi;
    }
}

template <int WM, int WN, int MTW, int RTW, int EPI, bool DB = false>
hipError_t launch_tile(GemmBatch& bt, hipStream_t stream) {
    auto kern = gemm_tile_kernel<WM, WN, MTW, RTW, EPI, DB>;
    constexpr size_t lds = tile_lds<WM, WN, MTW, RTW, DB>();
    if (lds > 65536) {
        static bool attr = false;
        if (!attr) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            attr = true;
        }
    }
    constexpr int TM = 16 * WM * MTW;
    const int n_mb = (bt.M + TM - 1) / TM;
    const int nks = EPI == EPI_PARTIAL ? bt.ksplit : 1;
    hipLaunchKernelGGL(kern, dim3(bt.total_tiles * n_mb * nks), dim3(WM * WN * kWave), lds,
                       stream, bt);
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

// The tiled store GEMM (128 x 128 tiles) serves bf16 from 384 input rows.  Measured at
// the 70B shape (512 rows): q/k/v 364 -> 191 us and the output projection 300 -> 192 us
// against the slice kernel.  Below 384 rows the slice kernel stays: with 64 x 64 tiles the
// dense tree's 256 rows took 63 / 65 us against 63 / 46, and 128 x 128 tiles leave most
// CUs idle there.
#ifndef MEDUSA_TILE_STORE
#define MEDUSA_TILE_STORE 1
#endif
#ifndef MEDUSA_TILE_SPLIT
#define MEDUSA_TILE_SPLIT 1
#endif
#ifndef MEDUSA_TILE_STORE_DB
#define MEDUSA_TILE_STORE_DB 1
#endif
#ifndef MEDUSA_TILE_STORE_CFG
#define MEDUSA_TILE_STORE_CFG 0
#endif
#ifndef MEDUSA_TILE_ARGMAX_CFG
#define MEDUSA_TILE_ARGMAX_CFG 0
#endif
#ifndef MEDUSA_TILE_SPLIT_ROWS
#define MEDUSA_TILE_SPLIT_ROWS 17
#endif
constexpr int kTileRtw = 4;
constexpr int kBigTile = 256;           // rows and columns of the sliced tiled kernel's tile
bool tile_store_eligible(medusa_dtype dt, int M, int K) {
    return MEDUSA_TILE_STORE && dt == MEDUSA_BF16 && M >= 384 && K % 64 == 0;
}
// The sliced 256 x 256 tiled kernel may run (bf16 from MEDUSA_TILE_SPLIT_ROWS input rows);
// partial_plan() decides whether it does.
bool tile_split_eligible(medusa_dtype dt, int M, int K) {
    return MEDUSA_TILE_SPLIT && dt == MEDUSA_BF16 && M >= MEDUSA_TILE_SPLIT_ROWS && K % 64 == 0;
}

template <int MT, int RT>
hipError_t launch_splitk_rows(GemmBatch& bt, hipStream_t stream) {
    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    hipLaunchKernelGGL((gemm_splitk_rows_kernel<MT, RT, MEDUSA_SPLIT_ROWS_PF>),
                       dim3(bt.total_tiles * n_mb), dim3(kThreads), 0, stream, bt);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_store(GemmBatch& bt, hipStream_t stream) {
    if (tile_store_eligible(sizeof(T) == 2 ? MEDUSA_BF16 : MEDUSA_F32, bt.M, bt.K))
    {
        constexpr bool DB = MEDUSA_TILE_STORE_DB != 0;
        if (MEDUSA_TILE_STORE_CFG == 1) return launch_tile<2, 2, 2 * kTileRtw, kTileRtw, EPI_STORE, DB>(bt, stream);
        if (MEDUSA_TILE_STORE_CFG == 2) return launch_tile<4, 2, kTileRtw, kTileRtw, EPI_STORE, DB>(bt, stream);
        return launch_tile<2, 2, kTileRtw, kTileRtw, EPI_STORE, DB>(bt, stream);
    }
    if (MEDUSA_SPLIT_ROWS && sizeof(T) == 2 && bt.K % (kSplitRowsChunk * kWaves) == 0) {
        if (bt.M <= 16) return launch_splitk_rows<1, 2>(bt, stream);
        if (bt.M <= 32) return launch_splitk_rows<2, 1>(bt, stream);
        return launch_splitk_rows<4, 1>(bt, stream);
    }
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
        case EPI_TYPICAL: return launch_mt<T, EPI_TYPICAL>(bt, stream);
        default: return launch_mt<T, EPI_ARGMAX>(bt, stream);
    }
}

}  // namespace

bool rowstream_eligible(medusa_dtype dt, int epi, int M, int K);

int gemm_rows_per_tile(medusa_dtype dt, int M, int epi, int K, int N) {
    if (epi == EPI_STORE && tile_store_eligible(dt, M, K)) return 32 * kTileRtw;
    if (epi == EPI_STORE) return 16 * splitk_rt(M);
    if (epi == EPI_PARTIAL) return kWavePartialRows;     // the tiled kernel: partial_tile_rows()
    if (rowstream_eligible(dt, epi, M, K)) {
        if (epi == EPI_TOPS) return kRsWavesTops * 16 * kRsRtw;
        return rs_small_vocab(M, N) ? kRsWavesSmallVocab * 16 * kRsRtwSmallVocab
                                    : kRsWavesArgmax * 16 * kRsRtwArgmax;
    }
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

// LDS bytes of a row-streaming workgroup: X chunk (plus a spare row slot), the waves' W
// tiles, the per-wave epilogue reductions.
template <int MT, int RTW, int CH, int NWV>
constexpr size_t rowstream_lds() {
    constexpr int XP = MEDUSA_RS_SWIZZLE && CH == 64 ? CH : CH + 8;
    return (size_t)(MT * 16 * XP + 8) * 2 + (size_t)NWV * 16 * RTW * XP * 2 +
           (size_t)NWV * MT * 16 * 8;
}

template <int MT, int EPI, int RTW, int PF, int CH, int NWV>
hipError_t launch_rowstream_t(GemmBatch& bt, hipStream_t stream) {
    auto kern = gemm_rowstream_kernel<MT, EPI, RTW, PF, CH, NWV>;
    constexpr size_t lds = rowstream_lds<MT, RTW, CH, NWV>();
    if (lds > 65536) {
        static bool attr = false;
        if (!attr) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            attr = true;
        }
    }
    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    hipLaunchKernelGGL(kern, dim3(bt.total_tiles * n_mb), dim3(NWV * kWave), lds, stream, bt);
    return hipGetLastError();
}

// Input-row blocks: up to 64 rows in one block of the smallest fitting size; above that,
// blocks of 128 rows.  Every block streams the workgroup's weight rows again, so larger
// blocks cut that traffic: against 64-row blocks the dense 256-node tree at the 8B shape
// verifies in 334 us instead of 469 (411 with a former kernel that staged the inputs in
// 512-column slabs), and batched 70B in 323 instead of 378.  256-row blocks need 240
// VGPRs, one workgroup per CU, and measured 384 us.
// Greedy verification past 64 rows runs on the tiled kernel, on the same 256-row weight
// tiles as the row-streaming kernel.  Up to 128 rows: 128 input rows per workgroup (2 x 4
// waves, two workgroups per CU).  Above: 256 input rows (4 x 4 waves, one workgroup per
// CU, LDS double-buffered), which halves the bytes each CU moves per flop: dense 256-node
// tree 320 -> 242 us, batched 70B 315 -> 233 us; at 128 rows the larger tile was slower
// (t(128) 940 -> 989 us per step), half of it being padding.
template <int EPI, int RTW, int PF, int CH, int NWV>
hipError_t launch_rowstream_m(GemmBatch& bt, hipStream_t stream) {
    if (bt.M <= 16) return launch_rowstream_t<1, EPI, RTW, PF, CH, NWV>(bt, stream);
    if (bt.M <= 32) return launch_rowstream_t<2, EPI, RTW, PF, CH, NWV>(bt, stream);
    if (bt.M <= 64) return launch_rowstream_t<4, EPI, RTW, PF, CH, NWV>(bt, stream);
    // the tiled kernel's weight rows per workgroup (WN * RTW * 16) are the tile size that
    // gemm_rows_per_tile() reports, which sizes the partials and the grid
    static_assert(EPI != EPI_ARGMAX || 4 * 4 * 16 == NWV * 16 * RTW, "argmax tile rows");
    if (EPI == EPI_ARGMAX)
    {
        if (bt.M <= 128) return launch_tile<2, 4, 4, 4, EPI_ARGMAX>(bt, stream);
        if (MEDUSA_TILE_ARGMAX_CFG == 1) return launch_tile<2, 4, 8, 4, EPI_ARGMAX, true>(bt, stream);
        if (MEDUSA_TILE_ARGMAX_CFG == 2) return launch_tile<4, 2, 4, 8, EPI_ARGMAX, true>(bt, stream);
        return launch_tile<4, 4, 4, 4, EPI_ARGMAX, true>(bt, stream);
    }
    return launch_rowstream_t<8, EPI, RTW, PF, CH, NWV>(bt, stream);
}

// Up to 64 rows over a small vocabulary: 4-wave workgroups of 16 weight rows each (64-row
// tiles).
template <int EPI, int PF, int CH>
hipError_t launch_rowstream_small_t(GemmBatch& bt, hipStream_t stream) {
    constexpr int W = kRsWavesSmallVocab, RT = kRsRtwSmallVocab;
    if (bt.M <= 16) return launch_rowstream_t<1, EPI, RT, PF, CH, W>(bt, stream);
    if (bt.M <= 32) return launch_rowstream_t<2, EPI, RT, PF, CH, W>(bt, stream);
    return launch_rowstream_t<4, EPI, RT, PF, CH, W>(bt, stream);
}
template <int EPI>
hipError_t launch_rowstream_small(GemmBatch& bt, hipStream_t stream) {
    constexpr int CH = MEDUSA_RS_CHUNK_SMALLV;
    if (bt.K % CH == 0) return launch_rowstream_small_t<EPI, MEDUSA_RS_PF_SMALLV, CH>(bt, stream);
    if (bt.K % kRsChunk != 0) return hipErrorInvalidValue;
    return launch_rowstream_small_t<EPI, 2, kRsChunk>(bt, stream);
}

hipError_t launch_rowstream(int epi, GemmBatch& bt, hipStream_t stream) {
    if (epi == EPI_TOPS)
        return bt.K % kRsChunkTops == 0
                   ? launch_rowstream_t<1, EPI_TOPS, kRsRtw, kRsPf, kRsChunkTops, kRsWavesTops>(bt, stream)
                   : launch_rowstream_t<1, EPI_TOPS, kRsRtw, kRsPf, kRsChunk, kRsWavesTops>(bt, stream);
    // the tile size follows each problem's width (gemm_rows_per_tile): one launch needs
    // them all on the same side
    int small = 0;
    for (int p = 0; p < bt.n_problems; ++p) small += rs_small_vocab(bt.M, bt.p[p].N) ? 1 : 0;
    if (small != 0 && small != bt.n_problems) return hipErrorInvalidValue;
    if (small)
        return epi == EPI_TYPICAL ? launch_rowstream_small<EPI_TYPICAL>(bt, stream)
                                  : launch_rowstream_small<EPI_ARGMAX>(bt, stream);
    if (epi == EPI_TYPICAL)
        return launch_rowstream_m<EPI_TYPICAL, kRsRtwArgmax, kRsPf, kRsChunk, kRsWavesArgmax>(bt, stream);
    return launch_rowstream_m<EPI_ARGMAX, kRsRtwArgmax, kRsPf, kRsChunk, kRsWavesArgmax>(bt, stream);
}

// Row-streaming MFMA path: bf16, contraction a multiple of 64, argmax or
// top-s epilogue (top-s only past the GEMV's two rows).
bool rowstream_eligible(medusa_dtype dt, int epi, int M, int K) {
    if (dt != MEDUSA_BF16 || K % kRsChunk != 0) return false;
    return epi == EPI_ARGMAX || epi == EPI_TYPICAL || (epi == EPI_TOPS && M > 2);
}

#ifndef MEDUSA_KSPLIT_WG
#define MEDUSA_KSPLIT_WG 384
#endif
#ifndef MEDUSA_CU_PF
#define MEDUSA_CU_PF 4
#endif
#ifndef MEDUSA_WAVE_PF
#define MEDUSA_WAVE_PF 2
#endif
constexpr int kPlanCus = 256;           // compute units the plan balances over (MI355X)
constexpr size_t kCuLdsBudget = 150 * 1024;

size_t cu_partial_lds(int nw, int K, int ks) {
    const int slice = K / ks;
    return (size_t)64 * (slice + 8) * 2 + (size_t)nw * 2 * 16 * kCuRt * (kCuChunk + 8) * 2;
}

PartialPlan partial_plan(medusa_dtype dt, int M, int K, const int* Ns, int n) {
    PartialPlan pl{0, 0, 0};
    if (dt != MEDUSA_BF16 || M <= 16 || K % kPartialChunk != 0) return pl;
    long long rows = 0;
    bool rows32 = true;
    for (int i = 0; i < n; ++i) {
        rows += Ns[i];
        rows32 = rows32 && Ns[i] % (16 * kCuRt) == 0;
    }
    // Both candidates are priced in the bytes the busiest CU moves: its rounds of weight and
    // input rows, its slice sums, and its share of the finalize pass.
    double best = -1;
    if (rows32 && K % kCuChunk == 0) {
        // one workgroup per CU, 64-row input blocks
        const int n_mb = (M + 63) / 64;
        static const int kWavesOpt[] = {2, 4, 6, 8};
        static const int kSplitOpt[] = {1, 2, 4, 8, 16};
        for (int nw : kWavesOpt)
            for (int ks : kSplitOpt) {
                if (K % (kCuChunk * ks) != 0 || cu_partial_lds(nw, K, ks) > kCuLdsBudget) continue;
                const long long R = 16LL * kCuRt * nw;
                const long long wgs = (rows + R - 1) / R * ks * n_mb;
                const long long rounds = (wgs + kPlanCus - 1) / kPlanCus;
                const double slice = (double)K / ks;
                const double per_wg = R * slice * 2 + 64 * slice * 2 + (ks > 1 ? R * 64 * 4 : 0);
                const double fin = ks > 1 ? (double)ks * M * rows * 4 / kPlanCus : 0;
                const double cost = rounds * per_wg + fin;
                if (best < 0 || cost < best) {
                    best = cost;
                    pl = PartialPlan{ks, nw, 0};
                }
            }
    }
    if (tile_split_eligible(dt, M, K)) {
        // 256 x 256 tiles (input rows past M cost no bandwidth: they read nothing new) in
        // as many contraction slices as fill the CUs best
        long long tiles = 0;
        for (int i = 0; i < n; ++i) tiles += (Ns[i] + kBigTile - 1) / kBigTile;
        tiles *= (M + kBigTile - 1) / kBigTile;
        const int chunks = K / 64;
        const double mv = std::min(M, kBigTile);
        for (int ks = 1; ks <= 16 && ks <= chunks; ++ks) {
            const long long rounds = (tiles * ks + kPlanCus - 1) / kPlanCus;
            const double slice = (double)((chunks + ks - 1) / ks) * 64;
            const double per_wg = (kBigTile + mv) * slice * 2;
            // one slice from 384 rows is the unsliced tiled store: no slice sums
            const bool sums = ks > 1 || !tile_store_eligible(dt, M, K);
            const double fin = sums ? 2.0 * ks * M * rows * 4 / kPlanCus : 0;
            const double cost = rounds * per_wg + fin;
            if (best < 0 || cost < best) {
                best = cost;
                pl = sums ? PartialPlan{ks, 0, 1} : PartialPlan{0, 0, 0};
            }
        }
    }
    if (best >= 0) return pl;
    // per-problem 64-row tiles on the single-wave kernel
    const int n_mb = (M + 63) / 64;
    long long tiles = 0;
    for (int i = 0; i < n; ++i) tiles += (Ns[i] + 63) / 64;
    const long long want = (MEDUSA_KSPLIT_WG + tiles * n_mb - 1) / (tiles * n_mb);
    pl.ksplit = (int)std::max(1LL, std::min(want, (long long)std::min(16, K / kPartialChunk)));
    return pl;
}

int partial_tile_rows(const PartialPlan& pl) { return pl.tile ? kBigTile : kWavePartialRows; }

template <int MT>
hipError_t launch_wave_partial(GemmBatch& bt, hipStream_t stream) {
    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    static_assert(kWavePartialRows == 16 * 4, "tile rows of the single-wave kernel");
    hipLaunchKernelGGL((gemm_wave_partial_kernel<MT, 4, MEDUSA_WAVE_PF, kPartialChunk>),
                       dim3(bt.total_tiles * n_mb * bt.ksplit), dim3(kWave), 0, stream, bt);
    return hipGetLastError();
}

template <int NW>
hipError_t launch_cu_partial(GemmBatch& bt, int rows, hipStream_t stream) {
    auto kern = gemm_cu_partial_kernel<NW, MEDUSA_CU_PF>;
    const size_t lds = cu_partial_lds(NW, bt.K, bt.ksplit);
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kCuLdsBudget);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int R = 16 * kCuRt * NW;
    const int n_mb = (bt.M + 63) / 64;
    hipLaunchKernelGGL(kern, dim3((rows + R - 1) / R * n_mb * bt.ksplit), dim3(NW * kWave), lds,
                       stream, bt, rows);
    return hipGetLastError();
}

hipError_t gemm_store_partial_launch(medusa_dtype dt, GemmBatch& bt, hipStream_t stream) {
    int Ns[kMaxProblems];
    int rows = 0;
    for (int p = 0; p < bt.n_problems; ++p) rows += (Ns[p] = bt.p[p].N);
    const PartialPlan pl = partial_plan(dt, bt.M, bt.K, Ns, bt.n_problems);
    if (pl.ksplit != bt.ksplit) return hipErrorInvalidValue;      // the caller sized part_val
    hipError_t e;
    if (pl.tile) {
        static_assert(16 * 4 * 4 == kBigTile, "sliced tile");
        e = launch_tile<4, 4, 4, 4, EPI_PARTIAL, true>(bt, stream);
    } else switch (pl.waves) {
    case 2: e = launch_cu_partial<2>(bt, rows, stream); break;
    case 4: e = launch_cu_partial<4>(bt, rows, stream); break;
    case 6: e = launch_cu_partial<6>(bt, rows, stream); break;
    case 8: e = launch_cu_partial<8>(bt, rows, stream); break;
    default:
        e = bt.M <= 16 ? launch_wave_partial<1>(bt, stream)
          : bt.M <= 32 ? launch_wave_partial<2>(bt, stream) : launch_wave_partial<4>(bt, stream);
    }
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
