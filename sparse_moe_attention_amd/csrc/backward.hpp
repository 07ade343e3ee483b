// Memory-bound kernels of the GQE backward pass (gradients of the layer in
// "Grouped Query Experts" explainer, technical summary, "Architecture and
// routing" and "Training and loss"; FrontiersMind GQE article, part 5):
//   * transpose_kernel: bf16 matrix transpose with zero padding (the weight
//     gradients contract over tokens, so their operands need tokens
//     contiguous);
//   * prep_kernel: per attention row, its output gradient (hard slot plus w
//     times the weighted slot), the weight gradient dw = <O, dC_weighted>,
//     delta = <dO, O>, and compact row-major and transposed copies of the
//     row's query and output gradient for the attention backward kernels;
//   * router_bwd_kernel: the router's logit gradients through the
//     renormalisation of the picked probabilities, the group softmax and the
//     load-balancing term;
//   * colsum_kernel / finalize_kernel: deterministic column sums (the router
//     bias gradient, the mean probabilities of the balancing loss);
//   * splitk_reduce_kernel: sums the split-K partial products of a weight
//     gradient in a fixed order and scatters row ranges to their buffers.
#pragma once

#include "gqe_common.hpp"

namespace gqe {

// Attention rows of one KV group, token by token: row = t*Rg + r, where Rg is
// k for a regular group and k+1 for the shared head's group s0 (its last row
// per token is the shared head). Each sequence of a group owns a padded run
// of rows (Lr regular, Lx for s0); groups follow each other in order.
struct RowSpace {
    int64_t T, Lr, Lx;
    int32_t Bt, R, s0;     // s0 < 0: no group carries an extra row
};
__host__ __device__ inline int rs_R(const RowSpace& s, int g) { return g == s.s0 ? s.R + 1 : s.R; }
__host__ __device__ inline int64_t rs_L(const RowSpace& s, int g) { return g == s.s0 ? s.Lx : s.Lr; }
__host__ __device__ inline int64_t rs_base(const RowSpace& s, int g, int b) {
    const int64_t before = (int64_t)s.Bt * ((int64_t)g * s.Lr + ((s.s0 >= 0 && g > s.s0) ? s.Lx - s.Lr : 0));
    return before + (int64_t)b * rs_L(s, g);
}

// ---------------------------------------------------------------------------
// Order of the attention-backward workgroups. Each (group, sequence) stream
// has a run of jobs of decreasing work; the regular streams (nrb of them) all
// have n_r jobs and the same work at the same index, the shared head's group
// (xb streams, one per sequence) has n_x jobs. Workgroups are issued in
// order of decreasing work across both classes: "level" l holds the extra
// jobs [P(l), P(l+1)) of every extra stream, then job l of every regular
// stream; a last level n_r holds the remaining extra jobs. P is the caller's
// split (P(0) = 0, P(n_r + 1) = n_x, non-decreasing). Workgroup i runs on
// XCD i % 8, so this order hands every XCD the same mix of long and short
// jobs; a fixed stream-to-XCD map would leave the XCD of the heavier class
// with about twice the work of the others.
// ---------------------------------------------------------------------------
struct BwdJob {
    int g, b;     // group and sequence
    int64_t j;    // job index within the stream (0 = the longest)
};
template <class Split>
__host__ __device__ inline int64_t bwd_job_count(int64_t l, int64_t nrb, int64_t xb, int64_t n_r, Split P) {
    return xb * P(l) + nrb * (l < n_r ? l : n_r);
}
template <class Split>
__host__ __device__ inline BwdJob bwd_job(int64_t L, const RowSpace& rs, int G, int64_t n_r, Split P) {
    const bool xc = rs.s0 >= 0;
    const int64_t xb = xc ? rs.Bt : 0, nrb = (int64_t)rs.Bt * (xc ? G - 1 : G);
    int64_t lo = 0, hi = n_r + 1;            // count(lo) <= L < count(hi)
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) / 2;
        if (bwd_job_count(mid, nrb, xb, n_r, P) <= L) lo = mid;
        else hi = mid;
    }
    const int64_t p = L - bwd_job_count(lo, nrb, xb, n_r, P);
    const int64_t nxl = xb * (P(lo + 1) - P(lo));
    BwdJob r;
    if (p < nxl) {
        r.g = rs.s0;
        r.b = (int)(p % rs.Bt);
        r.j = P(lo) + p / rs.Bt;
    } else {
        const int64_t u = p - nxl;
        const int gi = (int)(u / rs.Bt);
        r.g = (xc && gi >= rs.s0) ? gi + 1 : gi;
        r.b = (int)(u % rs.Bt);
        r.j = lo;
    }
    return r;
}
// Total jobs of both classes.
__host__ __device__ inline int64_t bwd_jobs(const RowSpace& rs, int G, int64_t n_r, int64_t n_x) {
    return (int64_t)rs.Bt * (rs.s0 >= 0 ? (int64_t)(G - 1) * n_r + n_x : (int64_t)G * n_r);
}
// dK/dV: job j of a stream is key tile j (BK keys), whose work is the rows
// from its first key on: (T - j*BK) * Rg. Extra job j goes before regular
// level l when its work is at least that of level l - 1.
struct DkdvSplit {
    int64_t T, BK, n;
    int R;
    __host__ __device__ int64_t operator()(int64_t l) const {
        if (l <= 0) return 0;
        if (l > n) return n;
        const int64_t f = (T + (l - 1) * BK * R) / (BK * (R + 1)) + 1;   // extra jobs at least as long as level l - 1
        return f < n ? f : n;
    }
};
// dQ: job j of a stream is its row tile counted from the last; regular and
// extra tiles that end at about the same token are about as long, so the
// extra jobs are spread in proportion, P(l) = l * n_x / n_r.
struct DqSplit {
    int64_t n_r, n_x;
    __host__ __device__ int64_t operator()(int64_t l) const {
        if (l <= 0) return 0;
        if (l > n_r) return n_x;
        return l * n_x / n_r;
    }
};

// ---------------------------------------------------------------------------
// dst[x][y] = src[y][x] for y < R, x < C; 0 elsewhere in the dst box
// [Co rows x Ro cols]. One 64x64 tile per workgroup through LDS: blockIdx.x
// = tile (ty + nty * tx), blockIdx.y steps src by zs and dst by zd elements.
// ---------------------------------------------------------------------------
struct TrArgs {
    const bf16* src;
    bf16* dst;
    int64_t lds, ldd;
    int64_t R, C, Ro, Co;
    int64_t zs, zd;
};

__global__ __launch_bounds__(256) void transpose_kernel(TrArgs a) {
    __shared__ bf16 tile[64][66];
    const int tid = threadIdx.x;
    const int64_t nty = (a.Ro + 63) / 64;
    const int64_t y0 = ((int64_t)blockIdx.x % nty) * 64, x0 = ((int64_t)blockIdx.x / nty) * 64;
    const bf16* src = a.src + (int64_t)blockIdx.y * a.zs;
    bf16* dst = a.dst + (int64_t)blockIdx.y * a.zd;
    const bool src_vec = ((reinterpret_cast<uintptr_t>(src) | (uintptr_t)(a.lds * 2)) & 15) == 0;
    const bool dst_vec = ((reinterpret_cast<uintptr_t>(dst) | (uintptr_t)(a.ldd * 2)) & 15) == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = tid + 256 * i, yy = u >> 3, xx = (u & 7) * 8;
        const int64_t y = y0 + yy, x = x0 + xx;
        bf16x8 v;
        if (y < a.R && x + 8 <= a.C && src_vec) {
            v = *reinterpret_cast<const bf16x8*>(src + y * a.lds + x);
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = (y < a.R && x + q < a.C) ? src[y * a.lds + x + q] : (bf16)0.f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) tile[yy][xx + q] = v[q];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = tid + 256 * i, xx = u >> 3, yy = (u & 7) * 8;
        const int64_t x = x0 + xx, y = y0 + yy;
        if (x >= a.Co) continue;
        bf16x8 v;
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = tile[yy + q][xx];
        if (y + 8 <= a.Ro && dst_vec) {
            *reinterpret_cast<bf16x8*>(dst + x * a.ldd + y) = v;
        } else {
            for (int q = 0; q < 8 && y + q < a.Ro; ++q) dst[x * a.ldd + y + q] = v[q];
        }
    }
}

// ---------------------------------------------------------------------------
// Per attention row: gathers the query and the output, forms the output
// gradient from the slot gradients dC = dout Wo:
//   routed row (g, r):  dO = dC_hard[g*k+r] + w[n,g,r] * dC_weighted,
//                       dw[n,g,r] = <O, dC_weighted>;
//   shared row:         dO = dC_shared;
// and delta = <dO, O> (with the bf16 dO the attention kernels use). Writes
// Q and dO row-major (rows of the row space), -delta, and for padding rows
// zero Q / dO / delta and a negated
// log-sum-exp of -inf (probability 0), so the attention kernels read whole
// tiles without tests.
// Grid: (row blocks of 64, G*Bt). 256 threads; d/8 lanes per row.
// ---------------------------------------------------------------------------
struct PrepArgs {
    const bf16* Qr;       // [N, G*k, d] routed queries (pre-scaled)
    const bf16* Qsh;      // [N, d]
    const bf16* C;        // [N, ldc] merged slots (O of every head)
    const bf16* dC;       // [N, ldc]
    const float* w;       // [N, G*k]
    bf16* Qc;             // [rows][d]
    bf16* dOc;
    float* lse;           // [rows] minus the log2 log-sum-exp (padding rows set here)
    float* dlt;           // [rows] minus delta
    float* dw;            // [N, G*k]
    RowSpace rs;
    int64_t ldc;
    int32_t G, k, d, wcol, shcol;   // weighted slot and shared slot column
};

template <int D>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int RPP = 256 / CPR;             // rows per pass
    const int tid = threadIdx.x;
    const int gb = blockIdx.y, g = gb / a.rs.Bt, b = gb % a.rs.Bt;
    const int Rg = rs_R(a.rs, g);
    const int64_t L = rs_L(a.rs, g), Lreal = a.rs.T * Rg;
    const int64_t rho0 = (int64_t)blockIdx.x * 64;
    if (rho0 >= L) return;
    const int64_t base = rs_base(a.rs, g, b);
    const int cc = tid % CPR;
    const int GK = a.G * a.k;
    for (int rr = tid / CPR; rr < 64; rr += RPP) {
        const int64_t rho = rho0 + rr;
        float q[8], o[8], dO[8];
        float s_dw = 0.f, s_dl = 0.f;
        int64_t n = 0;
        int r = 0;
        const bool real = rho < Lreal;
        if (real) {
            const int64_t t = rho / Rg;
            r = (int)(rho - t * Rg);
            n = (int64_t)b * a.rs.T + t;
            const bf16* crow = a.C + n * a.ldc;
            const bf16* dcrow = a.dC + n * a.ldc;
            if (r < a.k) {
                const int j = g * a.k + r;
                load8(a.Qr + (n * GK + j) * a.d + 8 * cc, q);
                load8(crow + (int64_t)j * a.d + 8 * cc, o);
                float dh[8], dwt[8];
                load8(dcrow + (int64_t)j * a.d + 8 * cc, dh);
                load8(dcrow + a.wcol + 8 * cc, dwt);
                const float wv = a.w[n * GK + j];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    dO[i] = (float)(bf16)(dh[i] + wv * dwt[i]);
                    s_dw += o[i] * dwt[i];
                }
            } else {
                load8(a.Qsh + n * a.d + 8 * cc, q);
                load8(crow + a.shcol + 8 * cc, o);
                load8(dcrow + a.shcol + 8 * cc, dO);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) s_dl += dO[i] * o[i];
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = dO[i] = 0.f;
        }
        // Row sums over the CPR lanes of the row (consecutive lanes).
#pragma unroll
        for (int m = 1; m < CPR; m <<= 1) {
            s_dw += __shfl_xor(s_dw, m);
            s_dl += __shfl_xor(s_dl, m);
        }
        if (cc == 0) {
            a.dlt[base + rho] = -s_dl;
            if (!real) a.lse[base + rho] = -INFINITY;
            else if (r < a.k) a.dw[n * GK + g * a.k + r] = s_dw;
        }
        store8(a.Qc + (base + rho) * a.d + 8 * cc, q);
        store8(a.dOc + (base + rho) * a.d + 8 * cc, dO);
    }
}

// ---------------------------------------------------------------------------
// Router backward, one thread per token. With p the per-group softmax of the
// logits, the picks' weights w = p_pick / S (S = sum of the token's G*k
// picked probabilities) and dw the gradient of w:
//   dp[g,m] = (dw[g,r] - sum(dw * w)) / S   if m is pick r of group g, else 0,
//           + coef * M * f[g,m] / (G * N)    (load-balancing term, f[g,m] =
//             count[g,m] / (N*k), the share of the group's picks),
//   dz[g,m] = p[g,m] * (dp[g,m] - sum_m' p[g,m'] dp[g,m']).
// Writes dz in fp32 (for the bias gradient) and bf16 into the gradient
// matrix dY at column lg_col, p in fp32 (for the balancing loss), and zeros
// into the padding columns [pad_col, ldy). (The d columns of the experts a
// token did not pick are zeroed by zero_cols_kernel.)
// ---------------------------------------------------------------------------
struct RouterBwdArgs {
    const float* logits;     // [N, E]
    const int32_t* idx;      // [N, G*k]
    const float* w;
    const float* dw;
    const int32_t* offsets;  // [E+1] expert segment starts: count[e] = offsets[e+1] - offsets[e]
    float* dz;               // [N, E]
    float* p;                // [N, E]
    bf16* dY;                // [N, ldy]
    int64_t N, ldy;
    int32_t G, M, k, d, lg_col, pad_col;
    float coef;
};

__global__ __launch_bounds__(64) void router_bwd_kernel(RouterBwdArgs a) {
    const int64_t n = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (n >= a.N) return;
    const int E = a.G * a.M, GK = a.G * a.k;
    const float* lg = a.logits + n * E;
    const int32_t* sel = a.idx + n * GK;
    const float* wv = a.w + n * GK;
    const float* dwv = a.dw + n * GK;
    bf16* dy = a.dY + n * a.ldy;
    float S = 0.f, sdw = 0.f;
    for (int g = 0; g < a.G; ++g) {
        float mx = -INFINITY;
        for (int m = 0; m < a.M; ++m) mx = fmaxf(mx, lg[g * a.M + m]);
        float den = 0.f;
        for (int m = 0; m < a.M; ++m) den += expf(lg[g * a.M + m] - mx);
        for (int r = 0; r < a.k; ++r) {
            S += expf(lg[g * a.M + sel[g * a.k + r]] - mx) / den;
            sdw += dwv[g * a.k + r] * wv[g * a.k + r];
        }
    }
    const float aux = a.coef * (float)a.M / ((float)a.G * (float)a.N * (float)a.N * (float)a.k);
    for (int g = 0; g < a.G; ++g) {
        float mx = -INFINITY;
        for (int m = 0; m < a.M; ++m) mx = fmaxf(mx, lg[g * a.M + m]);
        float den = 0.f;
        for (int m = 0; m < a.M; ++m) den += expf(lg[g * a.M + m] - mx);
        // dp of expert m and the group's sum p.dp
        auto dp_of = [&](int m, bool& picked) {
            const int e = g * a.M + m;
            float v = aux * (float)(a.offsets[e + 1] - a.offsets[e]);
            picked = false;
            for (int r = 0; r < a.k; ++r)
                if (sel[g * a.k + r] == m) {
                    v += (dwv[g * a.k + r] - sdw) / S;
                    picked = true;
                }
            return v;
        };
        float spdp = 0.f;
        for (int m = 0; m < a.M; ++m) {
            bool pk;
            spdp += expf(lg[g * a.M + m] - mx) / den * dp_of(m, pk);
        }
        for (int m = 0; m < a.M; ++m) {
            bool pk;
            const float pm = expf(lg[g * a.M + m] - mx) / den;
            const float dz = pm * (dp_of(m, pk) - spdp);
            const int e = g * a.M + m;
            a.dz[n * E + e] = dz;
            a.p[n * E + e] = pm;
            dy[a.lg_col + e] = (bf16)dz;
        }
    }
    for (int c = a.pad_col; c < a.ldy; ++c) dy[c] = (bf16)0.f;
}

// Column sums of two [N, E] fp32 matrices over a block of rows each:
// part[blk][e] and part[nblk + blk][e]. The G = 256 / E row lanes of a
// column (G*E threads) read interleaved rows, so every pass reads G whole
// consecutive rows; the lanes' sums are then added in lane order (fixed
// order: deterministic).
__global__ __launch_bounds__(256) void colsum_kernel(const float* a, const float* b, float* part, int64_t N, int E,
                                                     int rows_per_blk) {
    __shared__ float red[256];
    const int G = 256 / E;                     // row lanes per column (E <= 256)
    const int tid = threadIdx.x, e = tid % E, lr = tid / E;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_blk;
    const int64_t r1 = min<int64_t>(N, r0 + rows_per_blk);
    for (int m = 0; m < 2; ++m) {
        const float* src = m == 0 ? a : b;
        float s = 0.f;
        if (lr < G)
            for (int64_t r = r0 + lr; r < r1; r += G) s += src[r * E + e];
        red[tid] = s;
        __syncthreads();
        if (tid < E) {
            float t = 0.f;
            for (int i = 0; i < G; ++i) t += red[i * E + tid];
            part[((int64_t)m * gridDim.x + blockIdx.x) * E + tid] = t;
        }
        __syncthreads();
    }
}

// dbr[e] = sum of the dz partials; the balancing loss
// coef/G * sum_{g,m} M * f[g,m] * mean_n p[n,g,m]. The L = 256 / E lanes of
// expert e take partials i = lane, lane + L, ...; their sums are then added
// in lane order (deterministic).
__global__ __launch_bounds__(256) void finalize_kernel(const float* part, int nblk, const int32_t* offsets, int64_t N,
                                                       int G, int M, int k, float coef, float* dbr, float* aux_loss) {
    __shared__ float rz[256], rp[256], term[256];
    const int E = G * M, L = 256 / E, tid = threadIdx.x, e = tid % E, lane = tid / E;
    float sz = 0.f, sp = 0.f;
    if (lane < L)
        for (int i = lane; i < nblk; i += L) {
            sz += part[(int64_t)i * E + e];
            sp += part[(int64_t)(nblk + i) * E + e];
        }
    rz[tid] = sz;
    rp[tid] = sp;
    __syncthreads();
    if (tid < E) {
        float z = 0.f, q = 0.f;
        for (int l = 0; l < L; ++l) {
            z += rz[l * E + tid];
            q += rp[l * E + tid];
        }
        if (dbr != nullptr) dbr[tid] = z;
        const float f = (float)(offsets[tid + 1] - offsets[tid]) / ((float)N * (float)k);
        term[tid] = (float)M * f * (q / (float)N);
    }
    __syncthreads();
    if (tid == 0 && aux_loss != nullptr) {
        float s = 0.f;
        for (int i = 0; i < E; ++i) s += term[i];
        *aux_loss = coef * s / (float)G;
    }
}

// Zeroes columns [0, cols) of every row of a bf16 matrix (row stride ld,
// both multiples of 8): 16 bytes per thread, consecutive threads along a row.
__global__ __launch_bounds__(256) void zero_cols_kernel(bf16* m, int64_t rows, int64_t cols, int64_t ld) {
    const int64_t per = cols / 8, q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= rows * per) return;
    *reinterpret_cast<bf16x8*>(m + (q / per) * ld + (q % per) * 8) = bf16x8{};
}

// ---------------------------------------------------------------------------
// out_i[r][c] = sum_s part[s][row_begin_i + r][c] for each destination i, in
// split order. Four consecutive columns per thread.
// ---------------------------------------------------------------------------
struct RedDst {
    float* p;
    int64_t row_begin, n_rows;
};
struct RedArgs {
    const float* part;
    int64_t split_stride, rows, cols;
    int32_t n_split, n_dst;
    RedDst dst[6];
};

__global__ __launch_bounds__(256) void splitk_reduce_kernel(RedArgs a) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t cq = a.cols / 4;
    if (q >= a.rows * cq) return;
    const int64_t r = q / cq, c = (q % cq) * 4;
    f32x4 s = *reinterpret_cast<const f32x4*>(a.part + r * a.cols + c);
    for (int i = 1; i < a.n_split; ++i) s += *reinterpret_cast<const f32x4*>(a.part + i * a.split_stride + r * a.cols + c);
    for (int i = 0; i < a.n_dst; ++i) {
        const RedDst& d = a.dst[i];
        if (r >= d.row_begin && r < d.row_begin + d.n_rows) {
            float* o = d.p + (r - d.row_begin) * a.cols + c;
            if ((reinterpret_cast<uintptr_t>(o) & 15) == 0) {
                *reinterpret_cast<f32x4*>(o) = s;
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = s[v];
            }
        }
    }
}

}  // namespace gqe
