// Tile GEMM engine (C = A B^T, both operands K-contiguous) for the projection
// steps of the GQE layer, and the two kernels built on it:
//   * proj_gemm_kernel: one pass over x for several weight blocks at once
//     (dense K and V of every group, the shared head's Q, the router logits),
//     each block with its own output buffer and layout; also the output
//     projection and the dense-GQA Q projection;
//   * grouped_q_kernel: the sparse Q projection, one tile of one expert's
//     segment of the permutation per workgroup, rows gathered through the
//     permutation and scattered back to the dense [token, group, rank, d]
//     layout.
// Projections are dense contractions, so they run on MFMA: WM x WN waves, each wave a (BM/WM) x (BN/WN) block of 16x16 MFMA tiles;
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

template <typename T, int BM_, int BN_, int WM_, int WN_, int WPE_ = 2>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int WPE = WPE_;                    // waves per SIMD the registers are sized for
    static constexpr int BK = 128 / sizeof(T);          // K elements per 128-byte row
    static constexpr int VEC = 16 / sizeof(T);          // elements per 16-byte chunk
    static constexpr int FM = BM / (16 * WM);           // 16x16 blocks per wave, rows
    static constexpr int FN = BN / (16 * WN);           // 16x16 blocks per wave, cols
    static constexpr int NTH = WM * WN * 64;            // threads per workgroup
    static constexpr int RPP = NTH / 8;                  // tile rows loaded per pass (8 chunks a row)
    static constexpr int A_PER_THREAD = BM * 8 / NTH;   // 16-byte chunks each thread loads
    static constexpr int B_PER_THREAD = BN * 8 / NTH;
    static constexpr int A_BYTES = BM * kPitch;
    static constexpr int B_BYTES = BN * kPitch;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGE_BYTES;       // one stage; the second is an array of its own
    static_assert(WM * WN == 4 || WM * WN == 8, "4 or 8 waves");
    static_assert(BM * 8 % NTH == 0 && BN * 8 % NTH == 0, "tile rows must split over the threads");
};

// K loop. a_row[i] / b_row[i] point at the tile rows this thread loads
// (row tid/8 + RPP*i), already offset by its 16-byte column chunk. Every
// pointer must be readable for the whole K range: rows outside the problem
// point at some valid row instead (their results are never stored), so the
// loads need no branches. Tiles are staged with gfx950's direct global->LDS
// loads (global_load_lds_dwordx4): each lane fetches the global chunk that the
// swizzled layout puts in its LDS slot, so tiles never pass through
// registers. Stage kt+1 loads while stage kt computes; the two stages are
// separate LDS arrays, so the compiler does not make the reads of one wait
// for the loads into the other. A partial last K step zeroes the A chunks at
// or beyond K in LDS (their B chunks hold finite data from the row start).
// Leaves the C block of this wave in acc and the LDS free (all waves past the
// final barrier). In 16x16 block (i, j) of the wave a lane holds 4
// consecutive entries along one line of C: without SWAP, rows 4*(lane/16) ..
// +3 of column lane%16 (acc = A-block x B-block^T); with SWAP the transposed
// block, i.e. columns 4*(lane/16) .. +3 of row lane%16.
template <typename T, class Cfg, bool SWAP>
__device__ __forceinline__ void gemm_mainloop_dma(char* lds0, char* lds1, const T* const (&a_row)[Cfg::A_PER_THREAD],
                                                  const T* const (&b_row)[Cfg::B_PER_THREAD], int K,
                                                  f32x4 (&acc)[Cfg::FM][Cfg::FN]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const int c16 = tid & 7;
    const int cl = c16 ^ ((tid >> 3) & 7);                // logical chunk of this lane's slot (row & 7 = (tid/8) & 7)
    const int adj = (cl - c16) * Cfg::VEC;                 // the row pointers point at chunk c16
    const int nk = (K + Cfg::BK - 1) / Cfg::BK;
    static_assert(Cfg::RPP % 8 == 0, "slot rows keep their swizzle phase across passes");

#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto dma = [&](int kt, char* buf) {
        const bool kin = kt * Cfg::BK + cl * Cfg::VEC < K;
        const int ko = kin ? kt * Cfg::BK : 0;
#pragma unroll
        for (int i = 0; i < Cfg::A_PER_THREAD; ++i)
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(a_row[i] + adj + ko),
                                             (__attribute__((address_space(3))) void*)(buf + (Cfg::NTH * i + 64 * wave) * 16),
                                             16, 0, 0);
#pragma unroll
        for (int i = 0; i < Cfg::B_PER_THREAD; ++i)
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(b_row[i] + adj + ko),
                                             (__attribute__((address_space(3))) void*)(buf + Cfg::A_BYTES +
                                                                                     (Cfg::NTH * i + 64 * wave) * 16),
                                             16, 0, 0);
    };
    auto fix_k_tail = [&](int kt, char* buf) {
        if ((kt + 1) * Cfg::BK <= K) return;              // uniform
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (int s = tid; s < Cfg::BM * 8; s += Cfg::NTH) {
            const int r = s / 8, pc = s % 8;
            if (kt * Cfg::BK + (pc ^ (r & 7)) * Cfg::VEC >= K) st16(buf + r * kPitch + pc * 16, zero);
        }
        __syncthreads();
    };
    auto compute = [&](const char* As) {
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
                for (int j = 0; j < Cfg::FN; ++j)
                    acc[i][j] = SWAP ? mma16(bfg[j], af[i], acc[i][j]) : mma16(af[i], bfg[j], acc[i][j]);
        }
    };
    auto step = [&](int kt, char* cur, char* nxt) {
        fix_k_tail(kt, cur);
        if (kt + 1 < nk) dma(kt + 1, nxt);
        compute(cur);
        __syncthreads();   // releases cur and (waiting for the loads) publishes nxt
    };
    dma(0, lds0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, lds0, lds1);
        if (kt + 1 < nk) step(kt + 1, lds1, lds0);
    }
}

// The K loop over two STAGE_BYTES arrays.
template <typename T, class Cfg, bool SWAP>
__device__ __forceinline__ void gemm_kloop(char* lds0, char* lds1, const T* const (&a_row)[Cfg::A_PER_THREAD],
                                           const T* const (&b_row)[Cfg::B_PER_THREAD], int K,
                                           f32x4 (&acc)[Cfg::FM][Cfg::FN]) {
    gemm_mainloop_dma<T, Cfg, SWAP>(lds0, lds1, a_row, b_row, K, acc);
}

// ---------------------------------------------------------------------------
// Multi-block projection: out_s = A W_s^T for up to 4 weight blocks W_s laid
// side by side as one virtual weight matrix (block s starts at virtual column
// col_begin, a multiple of 8). A block whose output is transposed
// (OUT_HEADS_T) never shares a column tile with a row-major block: the host
// starts a block at a multiple of kProjClassAlign whenever the class changes.
// Each tile then writes straight from the accumulators, oriented so that a
// lane's four consecutive values run along the output's contiguous axis.
// ---------------------------------------------------------------------------
#ifndef GQE_PROJ_ALIGN
#define GQE_PROJ_ALIGN 128
#endif
constexpr int kProjClassAlign = GQE_PROJ_ALIGN;

// Four consecutive outputs from an accumulator, scaled (8 bytes bf16, 16
// fp32), as a non-temporal store: projection outputs are read by a later
// kernel, and keeping them out of L2 leaves it to the weight and activation
// tiles the GEMM re-reads (measured faster for the step as a whole).
template <typename T>
__device__ __forceinline__ void store4(T* o, const f32x4& v, float scale) {
    if constexpr (sizeof(T) == 2) {
        bf16x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = (bf16)(v[q] * scale);
        __builtin_nontemporal_store(__builtin_bit_cast(uint64_t, w), reinterpret_cast<uint64_t*>(o));
    } else {
        __builtin_nontemporal_store(v * scale, reinterpret_cast<f32x4*>(o));
    }
}
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
    // Split-K (weight gradients, whose contraction runs over every token):
    // n_split > 1 splits K into runs of k_split elements (a multiple of the
    // K step); split s reads A and W from element s*k_split on and writes its
    // partial product at out + s*split_stride (OUT_ROWS_F32 only, no bias).
    int32_t n_split;
    int32_t k_split;
    int32_t pad_;
    int64_t split_stride;
    ProjSeg seg[4];
};

template <typename T, class Cfg>
__device__ __forceinline__ void proj_tile(const ProjArgs& a, char* lds0, char* lds1, int64_t hw) {
    const int tid = threadIdx.x;
    const int64_t n_m = (a.M_rows + Cfg::BM - 1) / Cfg::BM;
    const int64_t tiles = n_m * a.n_tiles_n;
    const int ns = a.n_split > 1 ? a.n_split : 1;
    const int64_t L0 = xcd_logical_id(hw, tiles * ns);
    const int ksp = (int)(L0 / tiles);
    const int64_t L = L0 - (int64_t)ksp * tiles;
    const int64_t m0 = (L / a.n_tiles_n) * Cfg::BM;
    const int n0 = (int)(L % a.n_tiles_n) * Cfg::BN;
    const int koff = ns > 1 ? ksp * a.k_split : 0;
    const int Keff = ns > 1 ? min(a.k_split, a.K - koff) : a.K;
    const int64_t so = ns > 1 ? ksp * a.split_stride : 0;

    const T* a_row[Cfg::A_PER_THREAD];
    const T* b_row[Cfg::B_PER_THREAD];
#pragma unroll
    for (int i = 0; i < Cfg::A_PER_THREAD; ++i) {
        const int64_t r = m0 + tid / 8 + Cfg::RPP * i;
        a_row[i] = (const T*)a.A + (r < a.M_rows ? r : m0) * a.lda + koff + (tid & 7) * Cfg::VEC;
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_PER_THREAD; ++i) {
        const int vc = n0 + tid / 8 + Cfg::RPP * i;
        b_row[i] = (const T*)a.seg[0].W + koff + (tid & 7) * Cfg::VEC;   // columns past every block
        for (int s = 0; s < a.n_segs; ++s) {
            const int c = vc - a.seg[s].col_begin;
            if (c >= 0 && c < a.seg[s].n_cols)
                b_row[i] = (const T*)a.seg[s].W + (int64_t)c * a.K + koff + (tid & 7) * Cfg::VEC;
        }
    }
    static_assert(kProjClassAlign % Cfg::BN == 0, "a column tile holds one output class");

    // Sequence b and token t of tile row r (token row n = b*T + t), from one
    // division per tile.
    const int64_t b0 = m0 / a.T, t0 = m0 - b0 * a.T;
    auto split = [&](int r, int64_t& b, int64_t& t) {
        t = t0 + r;
        b = b0;
        while (t >= a.T) {
            t -= a.T;
            ++b;
        }
    };
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const int log2d = 31 - __builtin_clz(a.d);            // head widths are powers of two
    bool trans = false;
    for (int s = 0; s < a.n_segs; ++s)
        if (a.seg[s].col_begin <= n0 && n0 < a.seg[s].col_begin + a.seg[s].n_cols) trans = a.seg[s].mode == OUT_HEADS_T;
    f32x4 acc[Cfg::FM][Cfg::FN];
    // Fast path: every row of the tile is a token of one sequence, one block
    // covers all of the tile's columns, and vector stores are aligned; each
    // lane then stores its 16 quads at fixed offsets from one base pointer.
    int full_seg = -1;
    for (int s = 0; s < a.n_segs; ++s)
        if (a.seg[s].col_begin <= n0 && n0 + Cfg::BN <= a.seg[s].col_begin + a.seg[s].n_cols) full_seg = s;
    const bool fast = full_seg >= 0 && m0 + Cfg::BM <= a.M_rows && t0 + Cfg::BM <= a.T && (t0 & 3) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.seg[full_seg].out) & 15) == 0 &&
                      (a.seg[full_seg].mode == OUT_HEADS || a.seg[full_seg].mode == OUT_HEADS_T ||
                       (a.seg[full_seg].ld_out & 3) == 0) &&
                      (a.seg[full_seg].mode != OUT_ROWS_F32 || a.seg[full_seg].bias == nullptr);

    if (trans) {
        // Transposed heads: a lane holds tokens r .. r+3 of column c.
        gemm_kloop<T, Cfg, false>(lds0, lds1, a_row, b_row, Keff, acc);
        const int64_t ldo = (int64_t)a.Bt * a.Tpad;
        if (fast) {
            const ProjSeg& sg = a.seg[full_seg];
            const int c0 = n0 - sg.col_begin + wn * Cfg::FN * 16 + (lane & 15);
            T* p = (T*)sg.out + (int64_t)c0 * ldo + b0 * a.Tpad + t0 + wm * Cfg::FM * 16 + 4 * (lane >> 4);
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
                for (int i = 0; i < Cfg::FM; ++i) store4<T>(p + (int64_t)j * 16 * ldo + i * 16, acc[i][j], sg.scale);
            return;
        }
        for (int s = 0; s < a.n_segs; ++s) {
            const ProjSeg& sg = a.seg[s];
            if (sg.col_begin >= n0 + Cfg::BN || sg.col_begin + sg.n_cols <= n0) continue;
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j) {
                    const int c = n0 + (wn * Cfg::FN + j) * 16 + (lane & 15) - sg.col_begin;
                    const int r = (wm * Cfg::FM + i) * 16 + 4 * (lane >> 4);
                    if (c < 0 || c >= sg.n_cols || m0 + r >= a.M_rows) continue;
                    int64_t b, t;
                    split(r, b, t);
                    T* o = (T*)sg.out + (int64_t)c * ldo + b * a.Tpad + t;
                    if (t + 3 < a.T && m0 + r + 3 < a.M_rows && (t & 3) == 0) {
                        if constexpr (sizeof(T) == 2) {
                            bf16x4 w;
#pragma unroll
                            for (int v = 0; v < 4; ++v) w[v] = (bf16)(acc[i][j][v] * sg.scale);
                            *reinterpret_cast<bf16x4*>(o) = w;
                        } else {
                            *reinterpret_cast<f32x4*>(o) = acc[i][j] * sg.scale;
                        }
                    } else {
                        for (int v = 0; v < 4 && m0 + r + v < a.M_rows; ++v) {
                            int64_t bv, tv;
                            split(r + v, bv, tv);
                            ((T*)sg.out)[(int64_t)c * ldo + bv * a.Tpad + tv] = from_f32<T>(acc[i][j][v] * sg.scale);
                        }
                    }
                }
        }
        return;
    }

    // Row-major outputs: a lane holds columns c .. c+3 of row r.
    gemm_kloop<T, Cfg, true>(lds0, lds1, a_row, b_row, Keff, acc);
    if (fast) {
        const ProjSeg& sg = a.seg[full_seg];
        const int c0 = n0 - sg.col_begin + wn * Cfg::FN * 16 + 4 * (lane >> 4);
        const int r0 = wm * Cfg::FM * 16 + (lane & 15);
        if (sg.mode == OUT_ROWS) {
            T* p = (T*)sg.out + (m0 + r0) * sg.ld_out + c0;
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j) store4<T>(p + (int64_t)i * 16 * sg.ld_out + j * 16, acc[i][j], sg.scale);
        } else if (sg.mode == OUT_ROWS_F32) {   // no bias (checked above); split-K partial at offset so
            float* p = (float*)sg.out + so + (m0 + r0) * sg.ld_out + c0;
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j) {
                    float* o = p + (int64_t)i * 16 * sg.ld_out + j * 16;
                    if (ns > 1) *reinterpret_cast<f32x4*>(o) = acc[i][j] * sg.scale;   // read back at once: keep in L2
                    else store4<float>(o, acc[i][j], sg.scale);
                }
        } else {   // OUT_HEADS: token rows of one sequence, d-wide head rows
            const int64_t hstride = (int64_t)a.Bt * a.Tpad * a.d;
            T* p = (T*)sg.out + (b0 * a.Tpad + t0 + r0) * a.d;
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) {
                const int c = c0 + 16 * j;
                T* pj = p + (int64_t)(c >> log2d) * hstride + (c & (a.d - 1));
#pragma unroll
                for (int i = 0; i < Cfg::FM; ++i) store4<T>(pj + i * 16 * a.d, acc[i][j], sg.scale);
            }
        }
        return;
    }
    for (int s = 0; s < a.n_segs; ++s) {
        const ProjSeg& sg = a.seg[s];
        if (sg.col_begin >= n0 + Cfg::BN || sg.col_begin + sg.n_cols <= n0) continue;
        const bool vec_ok = (reinterpret_cast<uintptr_t>(sg.out) & 15) == 0 && (sg.mode == OUT_HEADS || (sg.ld_out & 3) == 0);
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) {
            const int r = (wm * Cfg::FM + i) * 16 + (lane & 15);
            const int64_t row = m0 + r;
            if (row >= a.M_rows) continue;
            int64_t b = 0, t = 0;
            if (sg.mode == OUT_HEADS) split(r, b, t);
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) {
                const int c = n0 + (wn * Cfg::FN + j) * 16 + 4 * (lane >> 4) - sg.col_begin;
                if (c < 0 || c >= sg.n_cols) continue;
                const f32x4 v = acc[i][j] * sg.scale;
                const bool full = c + 4 <= sg.n_cols;
                if (sg.mode == OUT_ROWS_F32) {
                    float* o = (float*)sg.out + so + row * sg.ld_out + c;
                    float w4[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) w4[q] = v[q] + ((sg.bias && c + q < sg.n_cols) ? sg.bias[c + q] : 0.f);
                    if (full && vec_ok) {
                        *reinterpret_cast<f32x4*>(o) = f32x4{w4[0], w4[1], w4[2], w4[3]};
                    } else {
                        for (int q = 0; q < 4 && c + q < sg.n_cols; ++q) o[q] = w4[q];
                    }
                    continue;
                }
                T* o = sg.mode == OUT_ROWS
                           ? (T*)sg.out + row * sg.ld_out + c
                           : (T*)sg.out + ((((int64_t)(c >> log2d)) * a.Bt + b) * a.Tpad + t) * a.d + (c & (a.d - 1));
                if (full && vec_ok) {
                    if constexpr (sizeof(T) == 2) {
                        bf16x4 w;
#pragma unroll
                        for (int q = 0; q < 4; ++q) w[q] = (bf16)v[q];
                        *reinterpret_cast<bf16x4*>(o) = w;
                    } else {
                        *reinterpret_cast<f32x4*>(o) = v;
                    }
                } else {
                    for (int q = 0; q < 4 && c + q < sg.n_cols; ++q) o[q] = from_f32<T>(v[q]);
                }
            }
        }
    }
}

// Persistent grid: workgroup b handles tiles b, b + gridDim.x, ... (grid a
// multiple of 8, so every tile index keeps its XCD), which lets one tile's
// stores drain while the next tile's K loop runs.
template <typename T, class Cfg>
__global__ __launch_bounds__(Cfg::NTH) __attribute__((amdgpu_waves_per_eu(Cfg::WPE, Cfg::WPE))) void proj_gemm_kernel(ProjArgs a) {
    // Two LDS stages, as separate arrays.
    __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
    __shared__ __attribute__((aligned(16))) char lds_b[Cfg::STAGE_BYTES];
    char* lds1 = lds_b;
    const int64_t n = ((a.M_rows + Cfg::BM - 1) / Cfg::BM) * a.n_tiles_n * (a.n_split > 1 ? a.n_split : 1);
    for (int64_t hw = blockIdx.x; hw < n; hw += gridDim.x) proj_tile<T, Cfg>(a, lds, lds1, hw);
}

// ---------------------------------------------------------------------------
// Projection of a handful of token rows (one decode step): out_s = A W_s^T
// for M_rows in the tens, where the time is one pass over the weights and
// the memory latency of that pass. Workgroup = 16 output columns x 16 rows
// (a.n_tiles_n = column blocks of 16). Its four waves take interleaved
// 32-wide K steps and issue the loads of up to eight steps at once, so each
// wave waits for memory about once per 256 elements of K; the four partial
// blocks are summed in LDS. W is the A operand of the product, so a lane ends
// with four consecutive output columns of one row. bf16, K a multiple of 32,
// row-major outputs only (OUT_ROWS, OUT_ROWS_F32 with its optional bias).
// ---------------------------------------------------------------------------
constexpr int kSkinnyRows = 16;

__device__ __forceinline__ f32x4 skinny_dot(const bf16* wrow, const bf16* xrow, int K, int wave, int q4) {
    const int S = K / 32;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = wave; s0 < S; s0 += 32) {
        Frag<bf16> wf[8], xf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = s0 + 4 * j;
            if (s < S) {
                wf[j] = ld_frag<bf16>(wrow + s * 32 + 8 * q4);
                xf[j] = ld_frag<bf16>(xrow + s * 32 + 8 * q4);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (s0 + 4 * j < S) acc = mma16(wf[j], xf[j], acc);
    }
    return acc;
}

// Sum of the four waves' blocks, left in wave 0 (the other waves return false).
__device__ __forceinline__ bool skinny_reduce(f32x4& acc, f32x4 (&part)[3][64], int wave, int lane) {
    if (wave > 0) part[wave - 1][lane] = acc;
    __syncthreads();
    if (wave > 0) return false;
    acc += part[0][lane];
    acc += part[1][lane];
    acc += part[2][lane];
    return true;
}

// (A template only so that the kernel is emitted in the one unit that
// instantiates it, with bf16.)
template <typename T>
__global__ __launch_bounds__(256) void skinny_proj_kernel(ProjArgs a) {
    static_assert(sizeof(T) == 2, "bf16 only");
    __shared__ f32x4 part[3][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    const int n0 = (int)(blockIdx.x % a.n_tiles_n) * 16;
    const int64_t m0 = (int64_t)(blockIdx.x / a.n_tiles_n) * kSkinnyRows;
    // Weight row of output column n0 + l16 (columns past every block read a
    // valid row whose results are dropped), activation row of token m0 + l16.
    const bf16* wrow = (const bf16*)a.seg[0].W;
    for (int s = 0; s < a.n_segs; ++s) {
        const int c = n0 + l16 - a.seg[s].col_begin;
        if (c >= 0 && c < a.seg[s].n_cols) wrow = (const bf16*)a.seg[s].W + (int64_t)c * a.K;
    }
    const int64_t m = m0 + l16;
    const bf16* xrow = (const bf16*)a.A + (m < a.M_rows ? m : m0) * a.lda;
    f32x4 acc = skinny_dot(wrow, xrow, a.K, wave, q4);
    if (!skinny_reduce(acc, part, wave, lane) || m >= a.M_rows) return;
    const int n = n0 + 4 * q4;   // a block starts at a multiple of 8: the four columns share it
    for (int s = 0; s < a.n_segs; ++s) {
        const ProjSeg& sg = a.seg[s];
        const int c = n - sg.col_begin;
        if (c < 0 || c >= sg.n_cols) continue;
        const f32x4 v = acc * sg.scale;
        if (sg.mode == OUT_ROWS_F32) {
            float* o = (float*)sg.out + m * sg.ld_out + c;
            for (int q = 0; q < 4 && c + q < sg.n_cols; ++q) o[q] = v[q] + (sg.bias ? sg.bias[c + q] : 0.f);
        } else {
            bf16* o = (bf16*)sg.out + m * sg.ld_out + c;
            if (c + 4 <= sg.n_cols && (sg.ld_out & 3) == 0 && (reinterpret_cast<uintptr_t>(sg.out) & 7) == 0) {
                bf16x4 w;
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q] = (bf16)v[q];
                *reinterpret_cast<bf16x4*>(o) = w;
            } else {
                for (int q = 0; q < 4 && c + q < sg.n_cols; ++q) o[q] = (bf16)v[q];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Sparse Q projection as a grouped GEMM. Expert e's picks form the segment
// [cbase[0][e], cbase[nC][e]) of the permutation, in token order; a
// workgroup takes BM consecutive rows of one segment (tile t of expert e),
// computes x[perm[i]] Wq_e^T for them and stores row i at row dst[i] of
// Qr [*, d]. Placement: workgroup hw runs on XCD x = hw % 8 and takes tile
// t = 8*(j / E) + x of expert j % E, j = hw / 8, so the E experts' tiles with
// the same index (about the same tokens, since every segment is in token
// order) run on one XCD and share x rows in its L2, and the non-empty tiles
// (small t) spread evenly over the XCDs. Tiles past the end of a segment exit.
// An expert is picked at most once per token, so ceil(N / BM) tiles bound
// every segment.
// ---------------------------------------------------------------------------
struct GroupArgs {
    const void* X;            // [N, K]
    const void* Wq;           // [E*d, K]
    void* Qr;                 // [N*G*k, d]
    const int32_t* perm;
    const int32_t* dst;
    const int32_t* cbase;     // [nC+1][E]: row 0 = segment starts, row nC = segment ends
    int64_t ldx;
    int32_t K;
    int32_t d;
    int32_t E;
    int32_t nC;
    int32_t n_t;              // tiles per expert (bound)
    float scale;              // multiplies the fp32 result before rounding
};

template <typename T, class Cfg>
__global__ __launch_bounds__(Cfg::NTH) __attribute__((amdgpu_waves_per_eu(Cfg::WPE, Cfg::WPE))) void grouped_q_kernel(GroupArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
    __shared__ __attribute__((aligned(16))) char lds_b[Cfg::STAGE_BYTES];
    char* lds1 = lds_b;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const int64_t j = blockIdx.x / 8;
    const int t = (int)(8 * (j / a.E) + blockIdx.x % 8), e = (int)(j % a.E);
    const int sb = a.cbase[e], se = a.cbase[(int64_t)a.nC * a.E + e];
    const int64_t rb64 = (int64_t)sb + (int64_t)t * Cfg::BM;
    if (rb64 >= se) return;
    const int rb = (int)rb64, re = min(se, rb + Cfg::BM);

    const T* b_row[Cfg::B_PER_THREAD];
#pragma unroll
    for (int i = 0; i < Cfg::B_PER_THREAD; ++i) {
        const int jj = tid / 8 + Cfg::RPP * i;
        b_row[i] = (const T*)a.Wq + ((int64_t)e * a.d + (jj < a.d ? jj : 0)) * a.K + (tid & 7) * Cfg::VEC;
    }
    const T* a_row[Cfg::A_PER_THREAD];
#pragma unroll
    for (int i = 0; i < Cfg::A_PER_THREAD; ++i) {
        const int r = rb + tid / 8 + Cfg::RPP * i;
        a_row[i] = (const T*)a.X + (int64_t)a.perm[r < re ? r : rb] * a.ldx + (tid & 7) * Cfg::VEC;
    }
    // Destination rows of the tile rows this lane stores, read before the K
    // loop so their latency hides behind it.
    int drows[Cfg::FM];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
        const int r = rb + (wm * Cfg::FM + i) * 16 + (lane & 15);
        drows[i] = r < re ? a.dst[r] : -1;
    }
    // Swapped operands: a lane holds output columns c .. c+3 of tile row r.
    f32x4 acc[Cfg::FM][Cfg::FN];
    gemm_kloop<T, Cfg, true>(lds, lds1, a_row, b_row, a.K, acc);
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
        const int drow = drows[i];
        if (drow < 0) continue;
#pragma unroll
        for (int jb = 0; jb < Cfg::FN; ++jb) {
            const int col = (wn * Cfg::FN + jb) * 16 + 4 * (lane >> 4);
            if (col >= a.d) continue;
            const f32x4 v = acc[i][jb] * a.scale;
            T* o = (T*)a.Qr + (int64_t)drow * a.d + col;
            if constexpr (sizeof(T) == 2) {
                bf16x4 w;
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q] = (bf16)v[q];
                *reinterpret_cast<bf16x4*>(o) = w;
            } else {
                *reinterpret_cast<f32x4*>(o) = v;
            }
        }
    }
}

}  // namespace gqe
