// Tile GEMM engine (C = A B^T, both operands K-contiguous) for the projection
// steps of the GQE layer, and the two kernels built on it:
//   * proj_gemm_kernel: one pass over x for several weight blocks at once
//     (dense K and V of every group, the shared head's Q, the router logits),
//     each block with its own output buffer and layout; also the output
//     projection and the dense-GQA Q projection;
//   * grouped_q_kernel: the sparse Q projection, one (token chunk, expert)
//     segment per workgroup, rows gathered through the permutation and
//     scattered back to the dense [token, group, rank, d] layout.
// Projections are dense contractions, so they run on MFMA: 256 threads as
// WM x WN waves, each wave a (BM/WM) x (BN/WN) block of 16x16 MFMA tiles;
// the K loop stages 128-byte rows of A and B through double-buffered LDS.
#pragma once

#include "gqe_common.hpp"

namespace gqe {

// LDS tile rows are 128 bytes (one K step), unpadded; the eight 16-byte
// chunks of row r are stored XOR-swizzled by r % 8, which keeps both the
// row-wise stores and the 16-lanes-down-a-column fragment reads free of bank
// conflicts on gfx950 (a 144-byte padded pitch measured 2-way conflicts).
constexpr int kPitch = 128;
__device__ __forceinline__ int tile_off(int r, int c) { return r * kPitch + ((c ^ (r & 7)) << 4); }

// Eight contraction elements of row r starting at chunk c (two chunks for fp32).
template <typename T> __device__ __forceinline__ Frag<T> ld_tile_frag(const char* base, int r, int c);
template <> __device__ __forceinline__ Frag<bf16> ld_tile_frag<bf16>(const char* base, int r, int c) {
    return ld_frag<bf16>(base + tile_off(r, c));
}
template <> __device__ __forceinline__ Frag<float> ld_tile_frag<float>(const char* base, int r, int c) {
    Frag<float> f;
    f.lo = *reinterpret_cast<const f32x4*>(base + tile_off(r, c));
    f.hi = *reinterpret_cast<const f32x4*>(base + tile_off(r, c + 1));
    return f;
}

template <typename T, int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int BK = 128 / sizeof(T);          // K elements per 128-byte row
    static constexpr int VEC = 16 / sizeof(T);          // elements per 16-byte chunk
    static constexpr int FM = BM / (16 * WM);           // 16x16 blocks per wave, rows
    static constexpr int FN = BN / (16 * WN);           // 16x16 blocks per wave, cols
    static constexpr int A_PER_THREAD = BM * 8 / 256;   // 16-byte chunks each thread loads
    static constexpr int B_PER_THREAD = BN * 8 / 256;
    static constexpr int A_BYTES = BM * kPitch;
    static constexpr int B_BYTES = BN * kPitch;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int SP = BN + 4;                   // fp32 pitch of the epilogue stage
    static constexpr int LDS_BYTES =
        (2 * STAGE_BYTES > BM * SP * 4) ? 2 * STAGE_BYTES : BM * SP * 4;
    static_assert(WM * WN == 4, "256 threads = 4 waves");
    static_assert(BM * 8 % 256 == 0 && BN * 8 % 256 == 0, "tile rows must split over 256 threads");
};

// K loop. a_row[i] / b_row[i] point at the tile rows this thread loads
// (row tid/8 + 32*i), already offset by its 16-byte column chunk; nullptr
// rows read as zeros, as do columns at or beyond K. Global loads run two K
// steps ahead of the MFMAs (two register sets), LDS holds two steps. Leaves
// the C block of this wave in acc and the LDS free (all waves past the final
// barrier).
template <typename T, class Cfg>
__device__ __forceinline__ void gemm_mainloop(char* lds, const T* const (&a_row)[Cfg::A_PER_THREAD],
                                              const T* const (&b_row)[Cfg::B_PER_THREAD], int K,
                                              f32x4 (&acc)[Cfg::FM][Cfg::FN]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const int c16 = tid & 7;
    const int nk = (K + Cfg::BK - 1) / Cfg::BK;
    u32x4 ra0[Cfg::A_PER_THREAD], rb0[Cfg::B_PER_THREAD];
    u32x4 ra1[Cfg::A_PER_THREAD], rb1[Cfg::B_PER_THREAD];
    const u32x4 zero = {0u, 0u, 0u, 0u};

#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto gload = [&](int kt, u32x4 (&ra)[Cfg::A_PER_THREAD], u32x4 (&rb)[Cfg::B_PER_THREAD]) {
        const int k0 = kt * Cfg::BK + c16 * Cfg::VEC;
        const bool kin = k0 < K;
#pragma unroll
        for (int i = 0; i < Cfg::A_PER_THREAD; ++i)
            ra[i] = (a_row[i] != nullptr && kin) ? ld16(a_row[i] + kt * Cfg::BK) : zero;
#pragma unroll
        for (int i = 0; i < Cfg::B_PER_THREAD; ++i)
            rb[i] = (b_row[i] != nullptr && kin) ? ld16(b_row[i] + kt * Cfg::BK) : zero;
    };
    auto sstore = [&](int buf, const u32x4 (&ra)[Cfg::A_PER_THREAD], const u32x4 (&rb)[Cfg::B_PER_THREAD]) {
        char* As = lds + buf * Cfg::STAGE_BYTES;
        char* Bs = As + Cfg::A_BYTES;
#pragma unroll
        for (int i = 0; i < Cfg::A_PER_THREAD; ++i) st16(As + tile_off(tid / 8 + 32 * i, c16), ra[i]);
#pragma unroll
        for (int i = 0; i < Cfg::B_PER_THREAD; ++i) st16(Bs + tile_off(tid / 8 + 32 * i, c16), rb[i]);
    };
    auto compute = [&](int buf) {
        const char* As = lds + buf * Cfg::STAGE_BYTES;
        const char* Bs = As + Cfg::A_BYTES;
#pragma unroll
        for (int ks = 0; ks < Cfg::BK / 32; ++ks) {
            const int kc = (ks * 32 + 8 * (lane >> 4)) * (int)sizeof(T) / 16;   // 16-byte chunk
            Frag<T> af[Cfg::FM], bfg[Cfg::FN];
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
                af[i] = ld_tile_frag<T>(As, (wm * Cfg::FM + i) * 16 + (lane & 15), kc);
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j)
                bfg[j] = ld_tile_frag<T>(Bs, (wn * Cfg::FN + j) * 16 + (lane & 15), kc);
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = mma16(af[i], bfg[j], acc[i][j]);
        }
    };
    // Step kt computes from LDS buffer kt%2, refills the register set that
    // held step kt with step kt+2, and moves step kt+1 (loaded one step ago)
    // from the other register set into LDS buffer (kt+1)%2.
    auto step = [&](int kt, u32x4 (&ra_kt)[Cfg::A_PER_THREAD], u32x4 (&rb_kt)[Cfg::B_PER_THREAD],
                    const u32x4 (&ra_n)[Cfg::A_PER_THREAD], const u32x4 (&rb_n)[Cfg::B_PER_THREAD]) {
        if (kt + 2 < nk) gload(kt + 2, ra_kt, rb_kt);
        compute(kt & 1);
        if (kt + 1 < nk) sstore((kt + 1) & 1, ra_n, rb_n);
        __syncthreads();
    };

    gload(0, ra0, rb0);
    if (nk > 1) gload(1, ra1, rb1);
    sstore(0, ra0, rb0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, ra0, rb0, ra1, rb1);
        if (kt + 1 < nk) step(kt + 1, ra1, rb1, ra0, rb0);
    }
}

// Writes this wave's C block to the fp32 LDS stage [BM][SP] and waits for
// all waves. Call after gemm_mainloop.
template <class Cfg>
__device__ __forceinline__ void stage_acc(float* stage, const f32x4 (&acc)[Cfg::FM][Cfg::FN]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = (wm * Cfg::FM + i) * 16 + 4 * (lane >> 4) + v;
                const int col = (wn * Cfg::FN + j) * 16 + (lane & 15);
                stage[row * Cfg::SP + col] = acc[i][j][v];
            }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Multi-block projection: out_s = A W_s^T for up to 4 weight blocks W_s laid
// side by side as one virtual weight matrix (block s starts at virtual column
// col_begin, a multiple of 8).
// ---------------------------------------------------------------------------
enum OutMode : int32_t {
    OUT_ROWS = 0,      // out[row * ld_out + col], type T
    OUT_ROWS_F32 = 1,  // out[row * ld_out + col] + bias[col], fp32
    OUT_HEADS = 2,     // per-head, per-sequence padded rows: out[((h*Bt + b)*Tpad + t)*d + c], type T
    OUT_HEADS_T = 3,   // transposed per head: out[(h*d + c)*(Bt*Tpad) + b*Tpad + t], type T
};

struct ProjSeg {
    const void* W;       // [n_cols, K]
    void* out;
    const float* bias;   // OUT_ROWS_F32 only, may be null
    int64_t ld_out;
    int32_t col_begin;
    int32_t n_cols;
    int32_t mode;
    float scale;         // multiplies the fp32 result before rounding (queries: log2(e)/sqrt(d))
};

struct ProjArgs {
    const void* A;       // [M_rows, K], row stride lda
    int64_t lda;
    int64_t M_rows;
    int64_t T, Tpad;     // token n = b*T + t (OUT_HEADS*)
    int32_t Bt;
    int32_t K;
    int32_t d;           // head width (OUT_HEADS*)
    int32_t n_segs;
    int32_t n_tiles_n;
    int32_t pad_;
    ProjSeg seg[4];
};

template <typename T, class Cfg>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void proj_gemm_kernel(ProjArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
    const int tid = threadIdx.x;
    const int64_t n_m = (a.M_rows + Cfg::BM - 1) / Cfg::BM;
    const int64_t L = xcd_logical_id(blockIdx.x, n_m * a.n_tiles_n);
    const int64_t m0 = (L / a.n_tiles_n) * Cfg::BM;
    const int n0 = (int)(L % a.n_tiles_n) * Cfg::BN;

    const T* a_row[Cfg::A_PER_THREAD];
    const T* b_row[Cfg::B_PER_THREAD];
#pragma unroll
    for (int i = 0; i < Cfg::A_PER_THREAD; ++i) {
        const int64_t r = m0 + tid / 8 + 32 * i;
        a_row[i] = r < a.M_rows ? (const T*)a.A + r * a.lda + (tid & 7) * Cfg::VEC : nullptr;
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_PER_THREAD; ++i) {
        const int vc = n0 + tid / 8 + 32 * i;
        b_row[i] = nullptr;
        for (int s = 0; s < a.n_segs; ++s) {
            const int c = vc - a.seg[s].col_begin;
            if (c >= 0 && c < a.seg[s].n_cols)
                b_row[i] = (const T*)a.seg[s].W + (int64_t)c * a.K + (tid & 7) * Cfg::VEC;
        }
    }
    f32x4 acc[Cfg::FM][Cfg::FN];
    gemm_mainloop<T, Cfg>(lds, a_row, b_row, a.K, acc);
    float* stage = reinterpret_cast<float*>(lds);
    stage_acc<Cfg>(stage, acc);

    // Row-vector modes: 8 consecutive columns of one row per item.
    constexpr int CCH = Cfg::BN / 8;
    for (int it = tid; it < Cfg::BM * CCH; it += 256) {
        const int r = it / CCH, cc = (it % CCH) * 8;
        const int64_t row = m0 + r;
        const int vc = n0 + cc;
        if (row >= a.M_rows) continue;
        for (int s = 0; s < a.n_segs; ++s) {
            const ProjSeg& sg = a.seg[s];
            const int c = vc - sg.col_begin;
            if (c < 0 || c >= sg.n_cols || sg.mode == OUT_HEADS_T) continue;
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = stage[r * Cfg::SP + cc + q] * sg.scale;
            const int nv = min(8, sg.n_cols - c);
            if (sg.mode == OUT_ROWS_F32) {
                float* o = (float*)sg.out + row * sg.ld_out + c;
                for (int q = 0; q < nv; ++q) o[q] = v[q] + (sg.bias ? sg.bias[c + q] : 0.f);
            } else {
                T* o;
                if (sg.mode == OUT_ROWS) {
                    o = (T*)sg.out + row * sg.ld_out + c;
                } else {  // OUT_HEADS
                    const int64_t b = row / a.T, t = row % a.T;
                    o = (T*)sg.out + (((int64_t)(c / a.d) * a.Bt + b) * a.Tpad + t) * a.d + (c % a.d);
                }
                if (nv == 8) {
                    store8<T>(o, v);
                } else {
                    for (int q = 0; q < nv; ++q) o[q] = from_f32<T>(v[q]);
                }
            }
        }
    }
    // Column-vector mode: 8 consecutive rows (tokens) of one column per item.
    constexpr int RCH = Cfg::BM / 8;
    for (int s = 0; s < a.n_segs; ++s) {
        const ProjSeg& sg = a.seg[s];
        if (sg.mode != OUT_HEADS_T) continue;
        for (int it = tid; it < Cfg::BN * RCH; it += 256) {
            const int cl = it / RCH, rr = (it % RCH) * 8;
            const int c = n0 + cl - sg.col_begin;
            if (c < 0 || c >= sg.n_cols) continue;
            const int64_t row = m0 + rr;
            if (row >= a.M_rows) continue;
            const int64_t b = row / a.T, t = row % a.T;
            T* o = (T*)sg.out + ((int64_t)(c / a.d) * a.d + (c % a.d)) * (a.Bt * a.Tpad) + b * a.Tpad + t;
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = stage[(rr + q) * Cfg::SP + cl] * sg.scale;
            if (row + 8 <= a.M_rows && t + 8 <= a.T && (t % 8) == 0) {
                store8<T>(o, v);
            } else {
                for (int q = 0; q < 8 && row + q < a.M_rows; ++q) {
                    const int64_t rq = row + q, bq = rq / a.T, tq = rq % a.T;
                    T* oq = (T*)sg.out + ((int64_t)(c / a.d) * a.d + (c % a.d)) * (a.Bt * a.Tpad) +
                            bq * a.Tpad + tq;
                    *oq = from_f32<T>(v[q]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Sparse Q projection as a grouped GEMM. Workgroup (chunk c, expert e)
// handles rows [cbase[c][e], cbase[c+1][e]) of expert e's segment of the
// permutation: the tokens of chunk c that picked e, in token order. Each
// row computes x[perm[i]] Wq_e^T and stores it at row dst[i] of Qr [*, d].
// ---------------------------------------------------------------------------
struct GroupArgs {
    const void* X;            // [N, K]
    const void* Wq;           // [E*d, K]
    void* Qr;                 // [N*G*k, d]
    const int32_t* perm;
    const int32_t* dst;
    const int32_t* cbase;     // [nC+1][E]
    int64_t ldx;
    int32_t K;
    int32_t d;
    int32_t E;
    int32_t nC;
    float scale;              // multiplies the fp32 result before rounding
};

template <typename T, class Cfg>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void grouped_q_kernel(GroupArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
    __shared__ int32_t s_dst[Cfg::BM];
    const int tid = threadIdx.x;
    const int64_t L = xcd_logical_id(blockIdx.x, (int64_t)a.nC * a.E);
    const int c = (int)(L / a.E), e = (int)(L % a.E);
    const int rb = a.cbase[(int64_t)c * a.E + e];
    const int re = a.cbase[(int64_t)(c + 1) * a.E + e];

    const T* b_row[Cfg::B_PER_THREAD];
#pragma unroll
    for (int i = 0; i < Cfg::B_PER_THREAD; ++i) {
        const int j = tid / 8 + 32 * i;
        b_row[i] = j < a.d ? (const T*)a.Wq + ((int64_t)e * a.d + j) * a.K + (tid & 7) * Cfg::VEC : nullptr;
    }
    for (int r0 = rb; r0 < re; r0 += Cfg::BM) {
        const T* a_row[Cfg::A_PER_THREAD];
#pragma unroll
        for (int i = 0; i < Cfg::A_PER_THREAD; ++i) {
            const int r = r0 + tid / 8 + 32 * i;
            a_row[i] = r < re ? (const T*)a.X + (int64_t)a.perm[r] * a.ldx + (tid & 7) * Cfg::VEC : nullptr;
        }
        for (int r = tid; r < Cfg::BM; r += 256) s_dst[r] = (r0 + r < re) ? a.dst[r0 + r] : -1;
        f32x4 acc[Cfg::FM][Cfg::FN];
        gemm_mainloop<T, Cfg>(lds, a_row, b_row, a.K, acc);
        float* stage = reinterpret_cast<float*>(lds);
        stage_acc<Cfg>(stage, acc);
        constexpr int CCH = Cfg::BN / 8;
        for (int it = tid; it < Cfg::BM * CCH; it += 256) {
            const int r = it / CCH, cc = (it % CCH) * 8;
            const int drow = s_dst[r];
            if (drow < 0 || cc >= a.d) continue;
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = stage[r * Cfg::SP + cc + q] * a.scale;
            store8<T>((T*)a.Qr + (int64_t)drow * a.d + cc, v);
        }
        __syncthreads();  // the stage and s_dst are reused by the next row tile
    }
}

}  // namespace gqe
