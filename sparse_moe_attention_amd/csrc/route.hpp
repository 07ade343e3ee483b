// Routing, permutation and weighted-slot kernels of the GQE layer.
//
// Routing ("Grouped Query Experts" explainer, technical summary, "Architecture
// and routing": per token a sparse subset of k experts of every group, and a
// renormalised weighted sum of their outputs; FrontiersMind GQE article,
// part 4: a light router scores every expert of every group and activates the
// best k, from the highest score down). Per token and group: softmax of the M
// logits in fp32, top-k by descending logit with ties to the lower index, and
// weights p_pick / (sum of p over all G*k picks of the token) -- or p_pick
// itself for the article's weighted-concatenation ablation (part 6).
//
// The permutation groups the (token, group, rank) picks by expert e = g*M + m
// so the sparse Q projection runs as one GEMM per expert segment. It is a
// stable counting sort in three passes, with tokens in chunks of 256:
//   route/hist: per-chunk histogram of experts (LDS atomics, exact counts);
//   scan:       per-expert prefix over chunks, then over experts -> the first
//               row of every (chunk, expert) piece and the segment offsets;
//   scatter:    each (chunk, expert) piece lists its tokens in token order.
// Nothing here is timing-dependent: the output is the same on every run.
#pragma once

#include "gqe_common.hpp"

namespace gqe {

constexpr int kChunk = 256;   // tokens per routing chunk (= workgroup size)

// One group of one token: the k best of its M logits (descending, ties to the
// lower index) and their softmax probabilities over the group.
__device__ inline void topk_group(const float* zg, int M, int k, int32_t* sel, float* prob) {
    float mx = -INFINITY;
    for (int m = 0; m < M; ++m) mx = fmaxf(mx, zg[m]);
    float se = 0.f;
    for (int m = 0; m < M; ++m) se += expf(zg[m] - mx);
    uint64_t taken = 0;
    for (int r = 0; r < k; ++r) {
        int best = -1;
        float bv = -INFINITY;
        for (int m = 0; m < M; ++m) {
            if ((taken >> m) & 1ull) continue;
            const float v = zg[m];
            if (best < 0 || v > bv) {   // strict: ties keep the lower index
                best = m;
                bv = v;
            }
        }
        taken |= 1ull << best;
        sel[r] = best;
        prob[r] = expf(bv - mx) / se;
    }
}

// MODE 0: route from fp32 logits [N, G*M] -> idx, w and the histogram
// (renorm = 0: w is the pick's probability, not renormalised).
// MODE 1: histogram of a caller-given idx (entries outside [0, M), and repeats
// of an earlier rank's expert in the same group, are skipped).
template <int MODE>
__global__ __launch_bounds__(256) void route_kernel(const float* logits, int32_t* idx, float* w,
                                                    int32_t* hist, int64_t N, int G, int M, int k, int renorm) {
    __shared__ int32_t h_lds[256];
    const int E = G * M;
    for (int e = threadIdx.x; e < E; e += 256) h_lds[e] = 0;
    __syncthreads();
    const int64_t n = (int64_t)blockIdx.x * kChunk + threadIdx.x;
    const int GK = G * k;
    if (n < N) {
        int32_t* irow = idx + n * GK;
        if (MODE == 0) {
            const float* z = logits + n * E;
            float* wrow = w + n * GK;
            float total = 0.f;
            for (int g = 0; g < G; ++g) {
                topk_group(z + g * M, M, k, irow + g * k, wrow + g * k);
                for (int r = 0; r < k; ++r) {
                    total += wrow[g * k + r];
                    atomicAdd(&h_lds[g * M + irow[g * k + r]], 1);
                }
            }
            if (renorm) {
                const float inv = 1.f / total;
                for (int q = 0; q < GK; ++q) wrow[q] = wrow[q] * inv;
            }
        } else {
            for (int g = 0; g < G; ++g)
                for (int r = 0; r < k; ++r) {
                    const int m = irow[g * k + r];
                    bool first = m >= 0 && m < M;          // out-of-range picks are skipped
                    for (int q = 0; q < r && first; ++q) first = irow[g * k + q] != m;   // so are repeats
                    if (first) atomicAdd(&h_lds[g * M + m], 1);
                }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) hist[(int64_t)blockIdx.x * E + e] = h_lds[e];
}

// One workgroup of 1024 threads. cbase [nC+1][E]: first permutation row of
// the picks of chunk c routed to expert e (row nC: segment ends). offsets
// [E+1]: segment starts. counts [E] (may be null): tokens per expert.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* hist, int32_t* cbase, int32_t* offsets,
                                                    int32_t* counts, int nC, int E) {
    __shared__ int32_t part[1024];
    __shared__ int32_t tot[256];
    __shared__ int32_t off[257];
    const int t = threadIdx.x;
    const int P = 1024 / E;                 // parts per expert column
    const int e = t % E, p = t / E;
    const int L = (nC + P - 1) / P;
    const int c0 = p * L, c1 = min(nC, c0 + L);
    if (p < P) {
        int sum = 0;
        for (int cc = c0; cc < c1; ++cc) sum += hist[(int64_t)cc * E + e];
        part[t] = sum;
    }
    __syncthreads();
    if (t < E) {
        int run = 0;
        for (int q = 0; q < P; ++q) {
            const int v = part[q * E + t];
            part[q * E + t] = run;
            run += v;
        }
        tot[t] = run;
    }
    __syncthreads();
    if (t == 0) {
        int o = 0;
        for (int q = 0; q < E; ++q) {
            off[q] = o;
            o += tot[q];
        }
        off[E] = o;
    }
    __syncthreads();
    if (t <= E) offsets[t] = off[t];
    if (counts != nullptr && t < E) counts[t] = tot[t];
    if (p < P) {
        int run = off[e] + part[t];
        for (int cc = c0; cc < c1; ++cc) {
            cbase[(int64_t)cc * E + e] = run;
            run += hist[(int64_t)cc * E + e];
        }
    }
    if (t < E) cbase[(int64_t)nC * E + t] = off[t] + tot[t];
}

// Workgroup = chunk of 256 tokens, thread = token. For every expert e the
// picks of the chunk are listed in token order at [cbase[c][e], ...): a
// token's rank is the number of earlier tokens of its wave that picked e
// (wave ballot) plus the totals of the earlier waves (one LDS exchange).
// perm = token, dst = row of the dense [N, G, k] layout (the first rank r at
// which the token picked e). Two passes over the experts: count, then write.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* idx, const int32_t* cbase, int32_t* perm,
                                                      int32_t* dst, int64_t N, int G, int M, int k) {
    __shared__ int32_t wtot[4][256];           // picks of expert e in each wave of the chunk
    const int E = G * M;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int64_t n = (int64_t)blockIdx.x * kChunk + tid;
    const bool valid = n < N;
    const int GK = G * k;
    const int32_t* row = idx + (valid ? n : 0) * GK;
    // r at which this token picked expert m of group g, or -1.
    auto pick_rank = [&](int g, int m) {
        int hit = -1;
        if (valid)
            for (int r = k - 1; r >= 0; --r)
                if (row[g * k + r] == m) hit = r;
        return hit;
    };
    for (int g = 0; g < G; ++g)
        for (int m = 0; m < M; ++m) {
            const uint64_t mask = __builtin_amdgcn_ballot_w64(pick_rank(g, m) >= 0);
            if ((tid & 63) == 0) wtot[wave][g * M + m] = __builtin_popcountll(mask);
        }
    __syncthreads();
    for (int g = 0; g < G; ++g)
        for (int m = 0; m < M; ++m) {
            const int r = pick_rank(g, m);
            const uint64_t mask = __builtin_amdgcn_ballot_w64(r >= 0);
            if (r < 0) continue;
            const int e = g * M + m;
            int pos = cbase[(int64_t)blockIdx.x * E + e];
            for (int w = 0; w < wave; ++w) pos += wtot[w][e];
            pos += __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
            perm[pos] = (int32_t)n;
            dst[pos] = (int32_t)(n * GK + g * k + r);
        }
}

// Weighted slot: C[n, GK*d + c] = sum_s w[n, s] * C[n, s*d + c] over the GK
// hard slots (fp32 accumulation). With scale_in_place (the weighted
// concatenation ablation) each hard slot is instead replaced by
// w[n, s] * C[n, s*d + c]. One thread per 8 columns of one token.
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(T* C, const float* w, int64_t N, int64_t ldc, int GK,
                                                      int d, int scale_in_place) {
    const int chunks = d / 8;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= N * chunks) return;
    const int64_t n = i / chunks;
    const int c = (int)(i % chunks) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    T* row = C + n * ldc;
    for (int s = 0; s < GK; ++s) {
        const float ws = w[n * GK + s];
        float v[8];
        load8<T>(row + s * d + c, v);
        if (scale_in_place) {
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] *= ws;
            store8<T>(row + s * d + c, v);
            continue;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += ws * v[q];
    }
    if (!scale_in_place) store8<T>(row + (int64_t)GK * d + c, acc);
}

}  // namespace gqe
