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
constexpr int kLdsXBytes = 32768;     // X chunk budget
constexpr int kUnroll = 4;            // k-steps whose W loads are issued together

template <typename T> constexpr int rt_for() { return sizeof(T) == 2 ? 4 : 2; }

template <typename T, int MT, int RT, int EPI>
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
    int pi = 0;
    while (pi + 1 < bt.n_problems && t >= bt.p[pi + 1].tile_begin) ++pi;
    const GemmProblem& P = bt.p[pi];
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
    const int KC = bt.KC;
    const int pitch = KC + 8;
    const T* X = static_cast<const T*>(P.X);

    for (int kc = 0; kc < K; kc += KC) {
        const int klen = min(KC, K - kc);
        __syncthreads();
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

        int ks = 0;
        for (; ks + 32 * kUnroll <= klen; ks += 32 * kUnroll) {
            Frag<T> wf[kUnroll][RT];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) wf[u][rt].load(wrow[rt] + kc + ks + 32 * u);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                Frag<T> xf[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int m = mt * 16 + ln;
                    if (m < Mb) xf[mt].load(xs + m * pitch + ks + 32 * u + 8 * lg);
                    else xf[mt].zero();
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) mma(acc[rt][mt], xf[mt], wf[u][rt]);
            }
        }
        for (; ks < klen; ks += 32) {
            Frag<T> wf[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) wf[rt].load(wrow[rt] + kc + ks);
            Frag<T> xf[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = mt * 16 + ln;
                if (m < Mb) xf[mt].load(xs + m * pitch + ks + 8 * lg);
                else xf[mt].zero();
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) mma(acc[rt][mt], xf[mt], wf[rt]);
        }
    }

    // acc[rt][mt][r] = Y[m0 + mt*16 + 4*lg + r][n_wave + rt*16 + ln]
    if (EPI == EPI_STORE) {
        T* out = static_cast<T*>(P.out);
        const T* bias = static_cast<const T*>(P.bias);
        const T* res = static_cast<const T*>(P.res);
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
        return;
    }

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
                reduce_best<16>(bv, bi);
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
                reduce_best<kWave>(bv, bi);
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

// k-way merge of the per-tile candidate lists (each sorted best first) into the top-s.
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(const MergeBatch bt) {
    __shared__ float sv[kWaves];
    __shared__ int si[kWaves];
    constexpr int kMaxOwned = 8;
    const int p = blockIdx.x / bt.M;
    const int m = blockIdx.x - p * bt.M;
    const MergeProblem& P = bt.p[p];
    const int s = P.s;
    const float* pv = P.part_val + (long long)m * P.n_tiles * s;
    const int32_t* pi = P.part_idx + (long long)m * P.n_tiles * s;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    int ptr[kMaxOwned];
    float hv[kMaxOwned];
    int hi[kMaxOwned];
#pragma unroll
    for (int j = 0; j < kMaxOwned; ++j) {
        const int tl = threadIdx.x + j * kThreads;
        ptr[j] = 0;
        if (tl < P.n_tiles) {
            hv[j] = pv[(long long)tl * s];
            hi[j] = pi[(long long)tl * s];
        } else {
            hv[j] = -INFINITY;
            hi[j] = INT_MAX;
        }
    }
    for (int round = 0; round < s; ++round) {
        float bv = -INFINITY;
        int bi = INT_MAX;
#pragma unroll
        for (int j = 0; j < kMaxOwned; ++j)
            if (better(hv[j], hi[j], bv, bi)) { bv = hv[j]; bi = hi[j]; }
        const int mine = bi;
        reduce_best<kWave>(bv, bi);
        if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
        __syncthreads();
        bv = sv[0];
        bi = si[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
        __syncthreads();
        if (threadIdx.x == 0) {
            P.out_ids[(long long)m * P.out_ld + round] = bi == INT_MAX ? -1 : bi;
            if (P.out_vals) P.out_vals[(long long)m * P.out_ld + round] = bv;
        }
        if (mine == bi && bi != INT_MAX) {
#pragma unroll
            for (int j = 0; j < kMaxOwned; ++j) {
                if (hi[j] == bi) {
                    const int tl = threadIdx.x + j * kThreads;
                    ++ptr[j];
                    if (ptr[j] < s) {
                        hv[j] = pv[(long long)tl * s + ptr[j]];
                        hi[j] = pi[(long long)tl * s + ptr[j]];
                    } else {
                        hv[j] = -INFINITY;
                        hi[j] = INT_MAX;
                    }
                }
            }
        }
    }
    for (int r = s + threadIdx.x; r < P.s_pad; r += kThreads) {
        P.out_ids[(long long)m * P.out_ld + r] = -1;
        if (P.out_vals) P.out_vals[(long long)m * P.out_ld + r] = 0.f;
    }
}

template <typename T, int MT, int EPI>
hipError_t launch_t(GemmBatch& bt, hipStream_t stream) {
    constexpr int RT = rt_for<T>();
    const int mrows = min(bt.M, MT * 16);
    int kc = (kLdsXBytes / (mrows * (int)sizeof(T)) - 8) / 32 * 32;
    kc = max(32, min(kc, (bt.K + 31) / 32 * 32));
    bt.KC = kc;
    size_t lds = (size_t)mrows * (kc + 8) * sizeof(T);
    if (EPI == EPI_TOPS) {
        const size_t need = (size_t)mrows * kWaves * RT * 16 * sizeof(float);
        if (need > lds) lds = need;
    }
    const int n_mb = (bt.M + MT * 16 - 1) / (MT * 16);
    dim3 grid(bt.total_tiles * n_mb);
    hipLaunchKernelGGL((gemm_kernel<T, MT, RT, EPI>), grid, dim3(kThreads), lds, stream, bt);
    return hipGetLastError();
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
        case EPI_STORE: return launch_mt<T, EPI_STORE>(bt, stream);
        case EPI_TOPS: return launch_mt<T, EPI_TOPS>(bt, stream);
        default: return launch_mt<T, EPI_ARGMAX>(bt, stream);
    }
}

}  // namespace

int gemm_rows_per_tile(medusa_dtype dt, int /*M*/, int /*epi*/) {
    return kWaves * 16 * (dt == MEDUSA_BF16 ? rt_for<bf16_t>() : rt_for<float>());
}

hipError_t gemm_launch(medusa_dtype dt, int epi, GemmBatch& bt, hipStream_t stream) {
    return dt == MEDUSA_BF16 ? launch_epi<bf16_t>(epi, bt, stream) : launch_epi<float>(epi, bt, stream);
}

hipError_t topk_merge_launch(const MergeBatch& bt, hipStream_t stream) {
    hipLaunchKernelGGL(topk_merge_kernel, dim3(bt.n_problems * bt.M), dim3(kThreads), 0, stream, bt);
    return hipGetLastError();
}

}  // namespace medusa
