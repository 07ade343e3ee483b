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

constexpr int kChunk = 256;   // tokens per routing chunk

// One group of one token: the k best of its M logits (descending, ties to the
// lower index) and their softmax probabilities over the group, passed to
// emit(r, m, p) in rank order. MM > 0: M == MM, and the logits are loaded
// once, all together, into registers; MM == 0: any M <= 64, read through zg.
// Both give the same values (same operations in the same order).
template <int MM, class Emit>
__device__ inline void topk_group(const float* zg, int M, int k, Emit&& emit) {
    float zr[MM > 0 ? MM : 1];
    if constexpr (MM > 0) {
#pragma unroll
        for (int m = 0; m < MM; ++m) zr[m] = zg[m];
    }
    auto z = [&](int m) -> float {
        if constexpr (MM > 0) return zr[m];
        else return zg[m];
    };
    const int Mg = MM > 0 ? MM : M;
    float mx = -INFINITY;
    for (int m = 0; m < Mg; ++m) mx = fmaxf(mx, z(m));
    float se = 0.f;
    for (int m = 0; m < Mg; ++m) se += expf(z(m) - mx);
    uint64_t taken = 0;
    for (int r = 0; r < k; ++r) {
        int best = -1;
        float bv = -INFINITY;
        for (int m = 0; m < Mg; ++m) {
            if ((taken >> m) & 1ull) continue;
            const float v = z(m);
            if (best < 0 || v > bv) {   // strict: ties keep the lower index
                best = m;
                bv = v;
            }
        }
        taken |= 1ull << best;
        emit(r, best, expf(bv - mx) / se);
    }
}

// Routing works on chunks of kChunk tokens with kRouteQ threads per token:
// thread (q, t) of a workgroup handles token t of the chunk and the groups
// [q*GQ, min(G, (q+1)*GQ)), GQ = ceil(G / kRouteQ), so each thread walks a
// quarter of the groups instead of all of them.
constexpr int kRouteQ = 4;
constexpr int kRouteThreads = kRouteQ * kChunk;
__host__ __device__ inline int route_gq(int G) { return (G + kRouteQ - 1) / kRouteQ; }

// The renormalisation denominator of a token: the picks' probabilities summed
// group by group (ranks in order) within each quarter of the groups, then the
// four quarter sums added in order. prob(g, r) returns pick r of group g.
template <class Prob>
__device__ inline float renorm_total(int G, int k, Prob&& prob) {
    const int gq = route_gq(G);
    float total = 0.f;
    for (int q = 0; q < kRouteQ; ++q) {
        float part = 0.f;
        for (int g = q * gq; g < min(G, (q + 1) * gq); ++g)
            for (int r = 0; r < k; ++r) part += prob(g, r);
        total += part;
    }
    return total;
}

// Caller-given picks (the training forward with injected routing): idx_in
// [N, G, k] is copied to idx, an entry outside [0, M) or repeating an
// earlier rank's expert in its group replaced by the group's lowest unused
// expert, so the picks stay a valid set; w gets the picks' group-softmax
// probabilities from the logits, renormalised over the token's G*k picks, in
// the router's own arithmetic (topk_group's max and sum, renorm_total's
// order). One thread per token.
__global__ __launch_bounds__(256) void inject_route_kernel(const float* __restrict__ logits,
                                                           const int32_t* __restrict__ idx_in,
                                                           int32_t* __restrict__ idx, float* __restrict__ w,
                                                           int64_t N, int G, int M, int k) {
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    const int E = G * M, GK = G * k;
    const float* z = logits + n * E;
    const int32_t* src = idx_in + n * GK;
    int32_t* irow = idx + n * GK;
    float* wrow = w + n * GK;
    for (int g = 0; g < G; ++g) {
        const float* zg = z + g * M;
        float mx = -INFINITY;
        for (int m = 0; m < M; ++m) mx = fmaxf(mx, zg[m]);
        float se = 0.f;
        for (int m = 0; m < M; ++m) se += expf(zg[m] - mx);
        uint64_t used = 0;
        for (int r = 0; r < k; ++r) {
            int m = src[g * k + r];
            if (m < 0 || m >= M || ((used >> m) & 1ull)) m = __builtin_ctzll(~used);   // k <= M: one is free
            used |= 1ull << m;
            irow[g * k + r] = m;
            wrow[g * k + r] = expf(zg[m] - mx) / se;
        }
    }
    const float inv = 1.f / renorm_total(G, k, [&](int g, int r) { return wrow[g * k + r]; });
    for (int j = 0; j < GK; ++j) wrow[j] *= inv;
}

// MODE 0: route from fp32 logits [N, G*M] -> idx, w and the histogram
// (renorm = 0: w is the pick's probability, not renormalised). MM as in
// topk_group. The quarter sums of renorm_total meet in LDS, so w is the same
// value renorm_total gives.
// MODE 1: histogram of a caller-given idx (entries outside [0, M), and repeats
// of an earlier rank's expert in the same group, are skipped).
template <int MODE, int MM>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float* __restrict__ logits,
                                                              int32_t* __restrict__ idx, float* __restrict__ w,
                                                              int32_t* __restrict__ hist, int64_t N, int G, int M,
                                                              int k, int renorm) {
    __shared__ int32_t h_lds[256];
    __shared__ float s_part[kRouteQ][kChunk];
    const int E = G * M;
    const int tid = threadIdx.x, q = tid / kChunk, t = tid % kChunk;
    for (int e = tid; e < E; e += kRouteThreads) h_lds[e] = 0;
    const int64_t n = (int64_t)blockIdx.x * kChunk + t;
    const int GK = G * k;
    const int gq = route_gq(G), g0 = q * gq, g1 = min(G, g0 + gq);
    const bool valid = n < N;
    if (MODE == 0) {
        const float* z = logits + (valid ? n : 0) * E;
        float part = 0.f;
        if (valid && renorm)
            for (int g = g0; g < g1; ++g) topk_group<MM>(z + g * M, M, k, [&](int, int, float p) { part += p; });
        s_part[q][t] = part;
    }
    __syncthreads();
    if (valid) {
        int32_t* irow = idx + n * GK;
        if (MODE == 0) {
            float* wrow = w + n * GK;
            float total = 0.f;
            for (int qq = 0; qq < kRouteQ; ++qq) total += s_part[qq][t];
            const float inv = renorm ? 1.f / total : 1.f;
            const float* z = logits + n * E;
            for (int g = g0; g < g1; ++g)
                topk_group<MM>(z + g * M, M, k, [&](int r, int m, float p) {
                    irow[g * k + r] = m;
                    wrow[g * k + r] = renorm ? p * inv : p;
                    atomicAdd(&h_lds[g * M + m], 1);
                });
        } else {
            for (int g = g0; g < g1; ++g)
                for (int r = 0; r < k; ++r) {
                    const int m = irow[g * k + r];
                    bool first = m >= 0 && m < M;          // out-of-range picks are skipped
                    for (int qq = 0; qq < r && first; ++qq) first = irow[g * k + qq] != m;   // so are repeats
                    if (first) atomicAdd(&h_lds[g * M + m], 1);
                }
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kRouteThreads) hist[(int64_t)blockIdx.x * E + e] = h_lds[e];
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

// Workgroup = chunk of kChunk tokens, kRouteQ threads per token as in
// route_kernel: waves 4q .. 4q+3 hold the chunk's tokens for the groups of
// quarter q, so every expert belongs to the waves of one quarter. For every
// expert e the picks of the chunk are listed in token order at
// [cbase[c][e], ...): a token's rank is the number of earlier tokens of its
// wave that picked e (wave ballot) plus the totals of the quarter's earlier
// waves (one LDS exchange). perm = token, dst = row of the dense [N, G, k]
// layout (the first rank r at which the token picked e). Two passes over the
// groups: count, then write; each takes a group's picks as a bit mask over its
// M experts (picks outside [0, M) are skipped, as route_kernel<1> skips them).
__global__ __launch_bounds__(kRouteThreads) void scatter_kernel(const int32_t* __restrict__ idx,
                                                                const int32_t* __restrict__ cbase,
                                                                int32_t* __restrict__ perm, int32_t* __restrict__ dst,
                                                                int64_t N, int G, int M, int k) {
    constexpr int WQ = kChunk / 64;            // waves per quarter
    __shared__ int32_t wtot[WQ][256];          // picks of expert e in each wave of its quarter
    __shared__ int32_t base[256];              // this chunk's first permutation row of each expert
    const int E = G * M;
    const int tid = threadIdx.x, q = tid / kChunk, t = tid % kChunk, wq = t >> 6;
    for (int e = tid; e < E; e += kRouteThreads) base[e] = cbase[(int64_t)blockIdx.x * E + e];
    const int64_t n = (int64_t)blockIdx.x * kChunk + t;
    const bool valid = n < N;
    const int GK = G * k;
    const int gq = route_gq(G), g0 = q * gq, g1 = min(G, g0 + gq);
    const int32_t* row = idx + (valid ? n : 0) * GK;
    auto group_mask = [&](int g) -> uint64_t {
        uint64_t pm = 0;
        if (valid) {
#pragma unroll 4
            for (int r = 0; r < k; ++r) {
                const int m = row[g * k + r];
                if (m >= 0 && m < M) pm |= 1ull << m;
            }
        }
        return pm;
    };
    for (int g = g0; g < g1; ++g) {
        const uint64_t pm = group_mask(g);
        for (int m = 0; m < M; ++m) {
            const uint64_t mask = __builtin_amdgcn_ballot_w64((pm >> m) & 1ull);
            if ((tid & 63) == 0) wtot[wq][g * M + m] = __builtin_popcountll(mask);
        }
    }
    __syncthreads();
    for (int g = g0; g < g1; ++g) {
        const uint64_t pm = group_mask(g);
        for (int m = 0; m < M; ++m) {
            const uint64_t mask = __builtin_amdgcn_ballot_w64((pm >> m) & 1ull);
            if (!((pm >> m) & 1ull)) continue;
            const int e = g * M + m;
            int pos = base[e];
            for (int w = 0; w < wq; ++w) pos += wtot[w][e];
            pos += __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
            int r = 0;
            while (row[g * k + r] != m) ++r;            // the first rank that picked m (bit set: one exists)
            perm[pos] = (int32_t)n;
            dst[pos] = (int32_t)(n * GK + g * k + r);
        }
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
    T* row = C + n * ldc;
    if (scale_in_place) {
        for (int s = 0; s < GK; ++s) {
            const float ws = w[n * GK + s];
            float v[8];
            load8<T>(row + s * d + c, v);
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] *= ws;
            store8<T>(row + s * d + c, v);
        }
        return;
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // Slots in ascending order; four slots' loads in flight at a time.
#pragma unroll 4
    for (int s = 0; s < GK; ++s) {
        const float ws = w[n * GK + s];
        float v[8];
        load8<T>(row + s * d + c, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += ws * v[q];
    }
    store8<T>(row + (int64_t)GK * d + c, acc);
}

}  // namespace gqe
