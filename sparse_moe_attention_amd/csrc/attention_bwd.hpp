// Causal flash-attention backward for the GQE layer: every picked expert and
// the shared head attend over their group's K/V ("Grouped Query Experts"
// explainer, technical summary, "Architecture and routing"; FrontiersMind GQE
// article, part 4), so the gradients of a group's K and V sum over all of
// the group's query rows, routed and shared.
//
// With scores s = q.k / sqrt(d), P the row softmax, dO the output gradient
// and delta = rowsum(dO * O):
//   dP = dO V^T,  dS = P * (dP - delta),
//   dV = P^T dO,  dK = dS^T q / sqrt(d),  dQ = dS K / sqrt(d).
// Queries are stored pre-scaled, Qs = q log2(e) / sqrt(d), and the forward
// saved -lse (lse = log2 of each row's normaliser), so P = exp2(Qs.k - lse)
// with no per-score arithmetic: -lse and -delta are the accumulators the
// score products start from. dK = ln(2) * dS^T Qs.
//
// Two kernels, no atomics (deterministic):
//   * attn_bwd_dkdv_kernel: one workgroup per (group, sequence, 128 keys),
//     two per CU;
//     each wave keeps 32 keys' K and V as resident MFMA operands and
//     accumulates their dK^T, dV^T over every query row at or after the
//     keys, 64 rows per step staged in LDS (Q and dO row-major, lse and
//     delta);
//   * attn_bwd_dq_kernel: one workgroup per (group, sequence, 128 rows: four
//     waves of 32), three per CU as in the forward; each wave keeps its 32
//     rows' Q and dO resident and
//     walks the key tiles up to its last token, staging K and V (row-major)
//     in LDS, accumulating dQ^T = K^T dS^T.
// The accumulations contract over rows (dK/dV) or keys (dQ), so their
// operands Q^T, dO^T and K^T are read from the same row-major LDS tiles with
// gfx950's transposing LDS read (ld_frag_tr): no transposed copies are made
// or staged.
// Score blocks are oriented so that the probabilities / score gradients a
// lane holds after the exponent are exactly the fragment the next product
// wants (no shuffles): the rows of a 16-row block are permuted so that the 8
// values a lane holds over a block pair are 8 consecutive rows (keys or
// queries), and the matching operand is one 16-byte LDS read.
#pragma once

#include <type_traits>

#include "attention.hpp"
#include "backward.hpp"

namespace gqe {

struct AttnBwdArgs {
    const bf16* Q;        // [rows][d], row space of RowSpace (pre-scaled queries)
    const bf16* dO;       // [rows][d]
    const float* lse;     // [rows] -lse, -inf on padding rows
    const float* dlt;     // [rows] -delta
    const bf16* K;        // [G][Bt][Tpad][d], zero beyond T
    const bf16* V;        // [G][Bt][Tpad][d], zero beyond T
    bf16* dY;             // [N][ldy] gradient matrix
    const int32_t* idx;   // [N][G*k]
    int64_t ldy;
    int64_t Tpad;
    RowSpace rs;
    int32_t G, M, k;
    int32_t colK, colV, colQsh;
    int32_t n_tiles;      // grid levels (key tiles / row tiles per sequence, the largest class)
};

// Tile shapes (the dK/dV kernel: keys per wave, waves, query rows per
// sub-step, waves per SIMD the registers are sized for; the dQ kernel: rows
// per wave, waves, keys per sub-step, waves per SIMD, keys per staged tile).
// The dQ kernel runs three four-wave workgroups per CU (64-key tiles keep
// their LDS at 32 KB, 32-key sub-steps their registers at 168): the waves
// sharing a SIMD then come from independent workgroups and overlap one
// another's exponent and product phases (10% faster than one eight-wave
// workgroup of 128-key tiles per CU at T = 32K). The dK/dV kernel runs two
// four-wave workgroups of 128 keys per CU (252 registers: two waves per
// SIMD), for the same reason: against one eight-wave workgroup of 256 keys
// per CU, whose staged Q/dO steps serve twice the keys, it measured 4.5%
// faster at T = 32K, 15% at T = 2048 and even at T = 1M, where the staged
// traffic had made the eight-wave form 20% faster while the transposed
// copies of Q and dO were staged as well.
#ifndef GQE_BWD_KW
#define GQE_BWD_KW 32
#endif
#ifndef GQE_BWD_NW
#define GQE_BWD_NW 4
#endif
#ifndef GQE_BWD_RS
#define GQE_BWD_RS 64
#endif
#ifndef GQE_BWD_WPE
#define GQE_BWD_WPE 2
#endif
#ifndef GQE_BWD_DQ_QW
#define GQE_BWD_DQ_QW 32
#endif
#ifndef GQE_BWD_DQ_NW
#define GQE_BWD_DQ_NW 4
#endif
#ifndef GQE_BWD_DQ_KS
#define GQE_BWD_DQ_KS 32
#endif
#ifndef GQE_BWD_DQ_WPE
#define GQE_BWD_DQ_WPE 3
#endif
#ifndef GQE_BWD_DQ_BKV
#define GQE_BWD_DQ_BKV 64
#endif
constexpr int kBwdKW = GQE_BWD_KW;         // keys per wave (dK/dV kernel)
// Waves per dK/dV workgroup (an eight-wave form exists for d = 64 only: head
// width 32 stages half the bytes per step, which 512 threads do not split
// evenly).
template <int D> constexpr int bwd_nw() { return D == 64 ? GQE_BWD_NW : 4; }
template <int D> constexpr int bwd_bk() { return kBwdKW * bwd_nw<D>(); }   // keys per dK/dV workgroup
constexpr int kBwdBKMax = kBwdKW * (GQE_BWD_NW > 4 ? GQE_BWD_NW : 4);
constexpr int kBwdQB = 64;                 // query rows per staged step (dK/dV kernel)
constexpr int kBwdRS = GQE_BWD_RS;         // rows per sub-step
// dQ kernel shapes: rows per wave, waves, keys per sub-step, waves per SIMD,
// keys per staged tile. Long sequences take one eight-wave workgroup of 256
// rows and 128-key tiles per CU: each staged K/V tile then serves twice the
// rows, which halves the K/V re-reads once a group's K/V no longer stays in
// the caches (T = 1M: 2.85 -> 2.59 s; 7% slower than the short shape at 32K).
template <int QW_, int NW_, int KS_, int WPE_, int BKV_>
struct DqShape {
    static constexpr int QW = QW_, NW = NW_, KS = KS_, WPE = WPE_, BKV = BKV_, BQ = NW_ * QW_;
    static_assert(QW % 16 == 0 && BKV % KS == 0 && KS % 32 == 0, "dQ tile shape");
};
using DqShort = DqShape<GQE_BWD_DQ_QW, GQE_BWD_DQ_NW, GQE_BWD_DQ_KS, GQE_BWD_DQ_WPE, GQE_BWD_DQ_BKV>;
using DqLong = DqShape<32, 8, 32, 2, 128>;
constexpr int kBwdDqBQMax = DqShort::BQ > DqLong::BQ ? DqShort::BQ : DqLong::BQ;
constexpr int kBwdBKVMax = DqShort::BKV > DqLong::BKV ? DqShort::BKV : DqLong::BKV;
static_assert(kBwdKW % 16 == 0 && kBwdQB % kBwdRS == 0 && kBwdRS % 32 == 0, "dK/dV tile shape");

// Row of a 64-row step held by row i of 16-row block qb (the same order as
// key_of_row): the 8 entries a lane holds over blocks 2j, 2j+1 are rows
// 32j + 8*(lane/16) .. +7.
__device__ __forceinline__ int qrow_of(int qb, int i) { return key_of_row(qb, i); }

// A operand of a product that contracts over 32 consecutive rows of a
// row-major bf16 LDS tile (rows r0 .. r0+31 of columns c0 .. c0+15, 16-byte
// chunks placed by k_chunk_off<CH>): lane (q4 = lane/16, i = lane%16) gets
// column c0 + i of rows r0 + 8*q4 .. +7, the layout that reading the
// transposed tile with one 16-byte load would give. gfx950's transposing
// read (ds_read_b64_tr_b16) hands lane i of each 16-lane group element i%4
// of the 8-byte reads of lanes 4e + i/4, e = 0..3 (lane layout checked on
// the device), so lane i reads 4 columns c0 + 4*(i%4) .. +3 of row
// r0 + 8*q4 + i/4, and once more 4 rows further for elements 4..7.
template <int CH>
__device__ __forceinline__ Frag<bf16> ld_frag_tr(const char* tile, int r0, int c0, int lane) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int q4 = lane >> 4, i = lane & 15;
    const int r = r0 + 8 * q4 + (i >> 2), c = c0 + 4 * (i & 3);
    const char* p0 = tile + k_chunk_off<CH>(r, c >> 3) + (c & 7) * 2;
    const char* p1 = tile + k_chunk_off<CH>(r + 4, c >> 3) + (c & 7) * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
    Frag<bf16> f;
    f.v = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
}

template <int D>
__global__ __launch_bounds__(bwd_nw<D>() * 64) __attribute__((amdgpu_waves_per_eu(GQE_BWD_WPE, GQE_BWD_WPE)))
void attn_bwd_dkdv_kernel(AttnBwdArgs a) {
    constexpr int NT = bwd_nw<D>() * 64;
    constexpr int kBwdBK = bwd_bk<D>();
    constexpr int KB = kBwdKW / 16;            // 16-key blocks per wave
    constexpr int DK = D / 32;                 // contraction steps over d
    constexpr int CB = D / 16;                 // 16-row blocks of dK^T / dV^T
    constexpr int QCH = D / 8;                 // 16-byte chunks per Q / dO row
    constexpr int QBS = kBwdRS / 16;           // 16-row blocks per sub-step
    constexpr int NSUB = kBwdQB / kBwdRS;
    constexpr int R_BYTES = kBwdQB * D * 2;    // one row-major tile
    constexpr int AUX = 1024;                  // lse (256 B), delta (256 B), padding
    constexpr int STAGE = 2 * R_BYTES + AUX;
    constexpr int R_PER_T = kBwdQB * QCH / NT;
    static_assert(kBwdQB * QCH % NT == 0, "tiles split evenly over the threads");
    __shared__ __attribute__((aligned(16))) char lds_a[STAGE];
    __shared__ __attribute__((aligned(16))) char lds_b[STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    // Workgroup -> (group, sequence, key tile), longest jobs first over both
    // row classes (bwd_job).
    const int64_t T_ = a.rs.T;
    const int64_t n_k = (T_ + kBwdBK - 1) / kBwdBK;
    const BwdJob job = bwd_job(blockIdx.x, a.rs, a.G, n_k, DkdvSplit{T_, kBwdBK, n_k, a.rs.R});
    const int g = job.g, b = job.b, kt = (int)job.j;
    const int k0 = kt * kBwdBK;
    if (k0 >= T_) return;
    const int Rg = rs_R(a.rs, g);
    const int64_t Lreal = T_ * Rg;
    const int64_t base = rs_base(a.rs, g, b);
    const int kw = k0 + wave * kBwdKW;                    // first key of this wave

    // Resident B operands: K^T and V^T fragments of the wave's keys
    // (column key = kw + 16kb + l16, contraction chunk 8*q4 of step dk).
    const bf16* Kg = a.K + ((int64_t)g * a.rs.Bt + b) * a.Tpad * D;
    const bf16* Vg = a.V + ((int64_t)g * a.rs.Bt + b) * a.Tpad * D;
    Frag<bf16> kf[KB][DK], vf[KB][DK];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            const int64_t off = (int64_t)(kw + 16 * kb + l16) * D + dk * 32 + 8 * q4;
            kf[kb][dk] = ld_frag<bf16>(Kg + off);
            vf[kb][dk] = ld_frag<bf16>(Vg + off);
        }
    f32x4 dkt[CB][KB], dvt[CB][KB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) dkt[cb][kb] = dvt[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Steps: 64-row blocks from the first row whose token reaches k0.
    const int64_t jb0 = ((int64_t)k0 * Rg) / kBwdQB;
    const int64_t jb1 = (Lreal + kBwdQB - 1) / kBwdQB;
    const int n_steps = (int)(jb1 - jb0);

    // Direct global->LDS staging; per-thread offsets relative to the step's first row.
    int roff[R_PER_T];
#pragma unroll
    for (int i = 0; i < R_PER_T; ++i) {
        const int s = tid + NT * i, r = s / QCH, p = s % QCH;
        roff[i] = r * D + (p ^ (((r & 3) | (((r >> 3) & 1) << 2)) & (QCH - 1))) * 8;
    }
    const bf16* Qb = a.Q + base * D;
    const bf16* dOb = a.dO + base * D;
    auto stage_ptr = [&](auto st) -> char* { return decltype(st)::value == 0 ? lds_a : lds_b; };
    auto dma = [&](int j, auto st) {
        const int64_t r0 = (jb0 + j) * kBwdQB;
        char* S = stage_ptr(st);
#pragma unroll
        for (int i = 0; i < R_PER_T; ++i) {
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(Qb + r0 * D + roff[i]),
                                             (__attribute__((address_space(3))) void*)(S + (NT * i + 64 * wave) * 16), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(dOb + r0 * D + roff[i]),
                                             (__attribute__((address_space(3))) void*)(S + R_BYTES + (NT * i + 64 * wave) * 16), 16, 0, 0);
        }
        if (wave == 0) {   // lanes 0-15: lse, 16-31: delta, 32-63: a copy of lse into the padding
            const float* src = (lane & 16) && lane < 32 ? a.dlt : a.lse;
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + base + r0 + 4 * (lane & 15)),
                                             (__attribute__((address_space(3))) void*)(S + 2 * R_BYTES), 16, 0, 0);
        }
    };

    // One sub-step of RS rows against the wave's keys; `masked` (uniform)
    // applies the causal test, which only sub-steps whose rows reach the
    // wave's keys need. (Inlined by force: an outlined call would keep the
    // accumulators it updates in scratch memory.)
    auto sub = [&](int64_t r0, int h, const char* Qs, const char* dOs, const char* aux,
                   bool masked) __attribute__((always_inline)) {
        f32x4 s[QBS][KB], dp[QBS][KB];
        f32x4 nls[QBS], ndl[QBS];
#pragma unroll
        for (int qq = 0; qq < QBS; ++qq) {
            const int qb = QBS * h + qq;
            const int chunk = 8 * (qb >> 1) + 2 * q4 + (qb & 1);   // rows 4*chunk .. +3
            nls[qq] = *reinterpret_cast<const f32x4*>(aux + 16 * chunk);
            ndl[qq] = *reinterpret_cast<const f32x4*>(aux + 256 + 16 * chunk);
        }
        // Score products 32 rows at a time (contraction steps inner for each
        // half): the exponent work of the first half can then overlap the
        // second half's products, and its dV/dK products the second half's
        // exponents.
#pragma unroll
        for (int hh = 0; hh < QBS / 2; ++hh)
#pragma unroll
        for (int dk = 0; dk < DK; ++dk)
#pragma unroll
            for (int qq = 2 * hh; qq < 2 * hh + 2; ++qq) {
                const int qr = qrow_of(QBS * h + qq, l16), c = 4 * dk + q4;
                const Frag<bf16> qf = ld_frag<bf16>(Qs + k_chunk_off<QCH>(qr, c));
                const Frag<bf16> of = ld_frag<bf16>(dOs + k_chunk_off<QCH>(qr, c));
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    s[qq][kb] = mma16(qf, kf[kb][dk], dk == 0 ? nls[qq] : s[qq][kb]);
                    dp[qq][kb] = mma16(of, vf[kb][dk], dk == 0 ? ndl[qq] : dp[qq][kb]);
                }
            }
        if (__builtin_expect(masked, false)) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                // rows of this sub-step before key*Rg (< 2^31 apart) are masked
                const int lim = (int)((int64_t)(kw + 16 * kb + l16) * Rg - r0);
#pragma unroll
                for (int qq = 0; qq < QBS; ++qq)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (qrow_of(QBS * h + qq, 4 * q4 + v) < lim) s[qq][kb][v] = -INFINITY;
            }
        }
        // P and dS fragments, 32 rows per contraction step: lane group q4
        // holds rows 32j + 8*q4 .. +7 of key column l16.
#pragma unroll
        for (int jj = 0; jj < QBS / 2; ++jj) {
            const int j32 = (QBS / 2) * h + jj;              // 32-row step within the 64 rows
#pragma unroll
            for (int qq = 2 * jj; qq < 2 * jj + 2; ++qq)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float pv = __builtin_amdgcn_exp2f(s[qq][kb][v]);
                        s[qq][kb][v] = pv;
                        dp[qq][kb][v] = pv * dp[qq][kb][v];
                    }
            Frag<bf16> pf[KB], sf[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    pf[kb].v[v] = (bf16)s[2 * jj][kb][v];
                    pf[kb].v[4 + v] = (bf16)s[2 * jj + 1][kb][v];
                    sf[kb].v[v] = (bf16)dp[2 * jj][kb][v];
                    sf[kb].v[4 + v] = (bf16)dp[2 * jj + 1][kb][v];
                }
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                // dO^T and Q^T: column cb*16 + l16, rows 32*j32 + 8*q4 .. +7
                const Frag<bf16> of = ld_frag_tr<QCH>(dOs, 32 * j32, cb * 16, lane);
                const Frag<bf16> qf = ld_frag_tr<QCH>(Qs, 32 * j32, cb * 16, lane);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    dvt[cb][kb] = mma16(of, pf[kb], dvt[cb][kb]);
                    dkt[cb][kb] = mma16(qf, sf[kb], dkt[cb][kb]);
                }
            }
        }
    };

    // One staged step. Edge steps (rows whose tokens reach the workgroup's
    // keys) test each sub-step for keys after every row (skip) or after some
    // row (causal mask); the others need neither and run branch-free.
    auto step = [&](int j, auto st, auto edge) __attribute__((always_inline)) {
        constexpr int SI = decltype(st)::value;
        if (j + 1 < n_steps) dma(j + 1, StageC<SI ^ 1>{});
        const int64_t r0 = (jb0 + j) * kBwdQB;
        const char* S = stage_ptr(st);
        const char* Qs = S;
        const char* dOs = S + R_BYTES;
        const char* aux = S + 2 * R_BYTES;
#pragma unroll
        for (int h = 0; h < NSUB; ++h) {       // rows RS*h .. RS*h + RS-1 of the step
            if constexpr (decltype(edge)::value) {
                // Row rho belongs to token floor(rho / Rg), and key > floor(rho / Rg)
                // exactly when rho < key * Rg: the causal tests need no division.
                const int64_t rlo = r0 + kBwdRS * h;
                if (rlo + kBwdRS - 1 < (int64_t)kw * Rg || rlo >= Lreal) continue;   // every key after every row's token
                sub(r0, h, Qs, dOs, aux, rlo < (int64_t)(kw + kBwdKW - 1) * Rg);
            } else {
                sub(r0, h, Qs, dOs, aux, false);
            }
        }
        __syncthreads();
    };

    if (n_steps > 0) {
        // Steps whose first row lies before the last key's first row are edge
        // steps; an even count keeps the two LDS stages in step with j.
        const int64_t thr = (int64_t)(k0 + kBwdBK - 1) * Rg;
        int jm = (int)min<int64_t>(n_steps, max<int64_t>(0, (thr + kBwdQB - 1) / kBwdQB - jb0));
        jm += jm & 1;
        dma(0, StageC<0>{});
        __syncthreads();
        for (int j = 0; j < jm; j += 2) {
            step(j, StageC<0>{}, std::true_type{});
            if (j + 1 < n_steps) step(j + 1, StageC<1>{}, std::true_type{});
        }
        for (int j = jm; j < n_steps; j += 2) {
            step(j, StageC<0>{}, std::false_type{});
            if (j + 1 < n_steps) step(j + 1, StageC<1>{}, std::false_type{});
        }
    }

    // dK = ln2 * dS^T Qs, dV = P^T dO: lane holds key kw + 16kb + l16,
    // columns 16cb + 4*q4 .. +3.
    constexpr float kLn2 = 0.69314718055994531f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int key = kw + 16 * kb + l16;
        if (key >= T_) continue;
        bf16* row = a.dY + ((int64_t)b * T_ + key) * a.ldy;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int c = g * D + cb * 16 + 4 * q4;
            bf16x4 wk, wv;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                wk[v] = (bf16)(dkt[cb][kb][v] * kLn2);
                wv[v] = (bf16)dvt[cb][kb][v];
            }
            *reinterpret_cast<bf16x4*>(row + a.colK + c) = wk;
            *reinterpret_cast<bf16x4*>(row + a.colV + c) = wv;
        }
    }
}

template <int D, class Shape>
__global__ __launch_bounds__(Shape::NW * 64) __attribute__((amdgpu_waves_per_eu(Shape::WPE, Shape::WPE)))
void attn_bwd_dq_kernel(AttnBwdArgs a) {
    constexpr int NT = Shape::NW * 64;
    constexpr int BKV = Shape::BKV;
    constexpr int QW = Shape::QW, BQ = Shape::BQ, KS = Shape::KS;
    constexpr int QBW = QW / 16;               // 16-row blocks per wave
    constexpr int KBS = KS / 16;               // 16-key blocks per sub-step
    constexpr int DK = D / 32;
    constexpr int CB = D / 16;
    constexpr int KCH = D / 8;                 // chunks per K / V row
    constexpr int K_BYTES = BKV * D * 2;
    constexpr int STAGE = 2 * K_BYTES;
    constexpr int K_PER_T = BKV * KCH / NT;
    static_assert(BKV * KCH % NT == 0, "tiles split evenly over the threads");
    __shared__ __attribute__((aligned(16))) char lds_a[STAGE];
    __shared__ __attribute__((aligned(16))) char lds_b[STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    // Workgroup -> (group, sequence, row tile counted from the last), longest
    // jobs first over both row classes (bwd_job).
    const int64_t T_ = a.rs.T;
    const int64_t n_r = (T_ * a.rs.R + BQ - 1) / BQ, n_x = (T_ * (a.rs.R + 1) + BQ - 1) / BQ;
    const BwdJob job = bwd_job(blockIdx.x, a.rs, a.G, n_r, DqSplit{n_r, n_x});
    const int g = job.g, b = job.b;
    const int Rg = rs_R(a.rs, g);
    const int64_t Lreal = T_ * Rg;
    const int n_t = (int)((Lreal + BQ - 1) / BQ);
    const int qt = n_t - 1 - (int)job.j;
    if (qt < 0) return;
    const int64_t base = rs_base(a.rs, g, b);
    const int64_t row0 = (int64_t)qt * BQ + wave * QW;    // first row of this wave

    const bf16* Qb = a.Q + base * D;
    const bf16* dOb = a.dO + base * D;
    Frag<bf16> qf[QBW][DK], of[QBW][DK];
    float nls[QBW], ndl[QBW];     // -lse, -delta of the lane's row (the score products' start)
    int tq[QBW];
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
        const int64_t rho = row0 + 16 * qb + l16;               // < L: padding rows are readable
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            qf[qb][dk] = ld_frag<bf16>(Qb + rho * D + dk * 32 + 8 * q4);
            of[qb][dk] = ld_frag<bf16>(dOb + rho * D + dk * 32 + 8 * q4);
        }
        nls[qb] = a.lse[base + rho];
        ndl[qb] = a.dlt[base + rho];
        tq[qb] = (int)(rho / Rg);
    }
    const int t_first = (int)(row0 / Rg);
    const int t_last = (int)min<int64_t>(T_ - 1, (row0 + QW - 1) / Rg);
    const int t_tile = (int)min<int64_t>(T_ - 1, ((int64_t)qt * BQ + BQ - 1) / Rg);
    const int n_kv = t_tile / BKV + 1;

    f32x4 dqt[CB][QBW];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) dqt[cb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const bf16* Kg = a.K + ((int64_t)g * a.rs.Bt + b) * a.Tpad * D;
    const bf16* Vg = a.V + ((int64_t)g * a.rs.Bt + b) * a.Tpad * D;
    int koff[K_PER_T];
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
        const int s = tid + NT * i, r = s / KCH, p = s % KCH;
        koff[i] = r * D + (p ^ (((r & 3) | (((r >> 3) & 1) << 2)) & (KCH - 1))) * 8;
    }
    auto stage_ptr = [&](auto st) -> char* { return decltype(st)::value == 0 ? lds_a : lds_b; };
    auto dma = [&](int j, auto st) {
        const int64_t k0 = (int64_t)j * BKV;
        char* S = stage_ptr(st);
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(Kg + k0 * D + koff[i]),
                                             (__attribute__((address_space(3))) void*)(S + (NT * i + 64 * wave) * 16), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(Vg + k0 * D + koff[i]),
                                             (__attribute__((address_space(3))) void*)(S + K_BYTES + (NT * i + 64 * wave) * 16), 16, 0, 0);
        }
    };

    // One sub-step of KS keys against the wave's rows; `masked` (uniform)
    // applies the causal test. (Inlined by force, as in the dK/dV kernel.)
    auto sub = [&](int k0, int h, const char* Ks, const char* Vs, bool masked) __attribute__((always_inline)) {
        f32x4 s[KBS][QBW], dp[KBS][QBW];
#pragma unroll
        for (int dk = 0; dk < DK; ++dk)
#pragma unroll
            for (int kb = 0; kb < KBS; ++kb) {
                const int kr = key_of_row(KBS * h + kb, l16), c = 4 * dk + q4;
                const Frag<bf16> kfr = ld_frag<bf16>(Ks + k_chunk_off<KCH>(kr, c));
                const Frag<bf16> vfr = ld_frag<bf16>(Vs + k_chunk_off<KCH>(kr, c));
#pragma unroll
                for (int qb = 0; qb < QBW; ++qb) {
                    const f32x4 c0 = {nls[qb], nls[qb], nls[qb], nls[qb]}, c1 = {ndl[qb], ndl[qb], ndl[qb], ndl[qb]};
                    s[kb][qb] = mma16(kfr, qf[qb][dk], dk == 0 ? c0 : s[kb][qb]);
                    dp[kb][qb] = mma16(vfr, of[qb][dk], dk == 0 ? c1 : dp[kb][qb]);
                }
            }
        if (__builtin_expect(masked, false)) {
#pragma unroll
            for (int kb = 0; kb < KBS; ++kb)
#pragma unroll
                for (int qb = 0; qb < QBW; ++qb)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (k0 + key_of_row(KBS * h + kb, 4 * q4 + v) > tq[qb]) s[kb][qb][v] = -INFINITY;
        }
#pragma unroll
        for (int kb = 0; kb < KBS; ++kb)
#pragma unroll
            for (int qb = 0; qb < QBW; ++qb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    s[kb][qb][v] = __builtin_amdgcn_exp2f(s[kb][qb][v]) * dp[kb][qb][v];
        // dS^T fragments: lane q4 holds keys 32kc + 8*q4 .. +7 of query l16.
#pragma unroll
        for (int kk = 0; kk < KBS / 2; ++kk) {
            const int kc = (KBS / 2) * h + kk;              // 32-key step within the tile
            Frag<bf16> sf[QBW];
#pragma unroll
            for (int qb = 0; qb < QBW; ++qb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    sf[qb].v[v] = (bf16)s[2 * kk][qb][v];
                    sf[qb].v[4 + v] = (bf16)s[2 * kk + 1][qb][v];
                }
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                // K^T: row cb*16 + l16 (a column of K), keys 32*kc + 8*q4 .. +7
                const Frag<bf16> ktf = ld_frag_tr<KCH>(Ks, 32 * kc, cb * 16, lane);
#pragma unroll
                for (int qb = 0; qb < QBW; ++qb) dqt[cb][qb] = mma16(ktf, sf[qb], dqt[cb][qb]);
            }
        }
    };

    // One staged key tile. Edge tiles (keys that reach the workgroup's first
    // token) test each sub-step for keys after every row of the wave (skip)
    // or after some row (causal mask); the others run branch-free.
    auto tile = [&](int j, auto st, auto edge) __attribute__((always_inline)) {
        constexpr int SI = decltype(st)::value;
        if (j + 1 < n_kv) dma(j + 1, StageC<SI ^ 1>{});
        const int k0 = j * BKV;
        const char* Ks = stage_ptr(st);
        const char* Vs = Ks + K_BYTES;
#pragma unroll
        for (int h = 0; h < BKV / KS; ++h) {     // keys KS*h .. KS*h + KS-1 of the tile
            if constexpr (decltype(edge)::value) {
                const int kh = k0 + KS * h;
                if (kh > t_last) continue;
                sub(k0, h, Ks, Vs, kh + KS - 1 > t_first);   // a key may lie above a row's token
            } else {
                sub(k0, h, Ks, Vs, false);
            }
        }
        __syncthreads();
    };

    // Tiles whose keys all precede the workgroup's first token need no causal
    // test; an even count keeps the two LDS stages in step with j.
    const int t_wg = (int)(((int64_t)qt * BQ) / Rg);
    int n_um = min(n_kv, (t_wg + 1) / BKV);
    n_um -= n_um & 1;
    dma(0, StageC<0>{});
    __syncthreads();
    for (int j = 0; j < n_um; j += 2) {
        tile(j, StageC<0>{}, std::false_type{});
        tile(j + 1, StageC<1>{}, std::false_type{});
    }
    for (int j = n_um; j < n_kv; j += 2) {
        tile(j, StageC<0>{}, std::true_type{});
        if (j + 1 < n_kv) tile(j + 1, StageC<1>{}, std::true_type{});
    }

    // dq = dS K / sqrt(d): lane holds row row0 + 16qb + l16, columns 16cb + 4*q4 .. +3.
    const float sc = 1.f / sqrtf((float)D);
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
        const int64_t rho = row0 + 16 * qb + l16;
        if (rho >= Lreal) continue;
        const int t = tq[qb], r = (int)(rho - (int64_t)t * Rg);
        const int64_t n = (int64_t)b * T_ + t;
        int col = a.colQsh;
        if (r < a.k) {
            const int m = a.idx[n * a.G * a.k + g * a.k + r];
            if (m < 0 || m >= a.M) continue;   // not a pick the forward can make: nothing to store
            col = (g * a.M + m) * D;
        }
        bf16* row = a.dY + n * a.ldy + col;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            bf16x4 w4;
#pragma unroll
            for (int v = 0; v < 4; ++v) w4[v] = (bf16)(dqt[cb][qb][v] * sc);
            *reinterpret_cast<bf16x4*>(row + cb * 16 + 4 * q4) = w4;
        }
    }
}

}  // namespace gqe

namespace gqe {

// ---------------------------------------------------------------------------
// Weight gradient of the routed query projections, grouped by expert over the
// forward's permutation (every picked expert owns its query projection,
// FrontiersMind GQE article, part 4, so its gradient sums over the tokens
// that picked it):
//   dWq[e*d + i][c] = sum over the tokens n of expert e's segment of
//                     dQ_e[n][i] * x[n][c],
// with dQ_e[n] read from the gradient matrix dY (columns e*d .. e*d + d - 1 of
// row n) and x[n] from the layer input. Only the G*k picks per token enter,
// not the M experts' columns of dY (zero where unpicked). The contraction
// runs over gathered tokens, so both operands are staged token-major and
// their MFMA fragments come from the transposing LDS read (ld_frag_tr).
// Workgroup = (split s, expert e, column tile ct): tokens of split s of the
// expert's segment against 256 columns of x (four waves of 64 x 64; 80 KB of
// LDS, two workgroups per CU; 64 x 128 tiles at three per CU measured 1-4%
// slower); every workgroup writes its fp32
// partial to part[s] (zeros for an empty split), and splitk_reduce_kernel
// sums the splits in a fixed order (deterministic).
// ---------------------------------------------------------------------------
struct GroupDwArgs {
    const bf16* dY;        // [N][ldy]
    const bf16* X;         // [N][D]
    const int32_t* perm;   // permutation row -> token
    const int32_t* cbase;  // [nC+1][E]: row 0 = segment starts, row nC = segment ends
    float* part;           // [S][E*d][D]
    int64_t ldy, split_stride;
    int32_t D, E, nC, S, n_ct;
};
constexpr int kDwBN = 256;     // x columns per workgroup (64 per wave)
constexpr int kDwBK = 64;      // tokens per staged step

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void grouped_dw_kernel(GroupDwArgs a) {
    constexpr int NT = 256;
    constexpr int QCH = D / 8;                 // 16-byte chunks per dQ row
    constexpr int XCH = kDwBN / 8;             // 16-byte chunks per staged x row
    constexpr int Q_BYTES = kDwBK * D * 2;
    constexpr int X_BYTES = kDwBK * kDwBN * 2;
    constexpr int STAGE = Q_BYTES + X_BYTES;
    constexpr int Q_PER_T = kDwBK * QCH / NT;
    constexpr int X_PER_T = kDwBK * XCH / NT;
    constexpr int FM = D / 16;                 // 16-row blocks of the d rows
    constexpr int FN = 4;                      // 16-column blocks per wave
    static_assert(kDwBK * QCH % NT == 0 && kDwBK * XCH % NT == 0 && kDwBN == 4 * FN * 16, "dW tile shape");
    __shared__ __attribute__((aligned(16))) char lds_a[STAGE];
    __shared__ __attribute__((aligned(16))) char lds_b[STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ct = (int)(blockIdx.x % a.n_ct);
    const int e = (int)((blockIdx.x / a.n_ct) % a.E);
    const int s = (int)(blockIdx.x / ((int64_t)a.n_ct * a.E));
    const int c0 = ct * kDwBN;
    const int sb = a.cbase[e], se = a.cbase[(int64_t)a.nC * a.E + e];
    const int len = se - sb;
    const int per = ((len + a.S - 1) / a.S + kDwBK - 1) / kDwBK * kDwBK;   // whole steps per split
    const int p0 = sb + min(len, s * per), p1 = sb + min(len, (s + 1) * per);
    const int n_steps = (p1 - p0 + kDwBK - 1) / kDwBK;

    // Staged chunks of this thread: slot it = tid + NT*i holds chunk it % CH of
    // row it / CH, which is the row's logical chunk (it % CH) ^ swz(row).
    auto swz = [](int r) { return (r & 3) | (((r >> 3) & 1) << 2); };
    int q_off[Q_PER_T], x_off[X_PER_T];
#pragma unroll
    for (int i = 0; i < Q_PER_T; ++i) {
        const int it = tid + NT * i, r = it / QCH;
        q_off[i] = e * D + ((it % QCH) ^ (swz(r) & (QCH - 1))) * 8;
    }
#pragma unroll
    for (int i = 0; i < X_PER_T; ++i) {
        const int it = tid + NT * i, r = it / XCH;
        const int c = c0 + ((it % XCH) ^ (swz(r) & (XCH - 1))) * 8;
        x_off[i] = c < a.D ? c : 0;            // columns past D: any valid column, never stored
    }
    // Tokens of this thread's staged rows for the next step to load (rows
    // past the split repeat its first token; their dQ rows are zeroed in LDS
    // before use). Fetched one step ahead of their use, so the gathers never
    // wait on the permutation.
    int tq[Q_PER_T], tx[X_PER_T];
    auto fetch_tokens = [&](int j) {
#pragma unroll
        for (int i = 0; i < Q_PER_T; ++i) {
            const int p = p0 + j * kDwBK + (tid + NT * i) / QCH;
            tq[i] = a.perm[p < p1 ? p : p0];
        }
#pragma unroll
        for (int i = 0; i < X_PER_T; ++i) {
            const int p = p0 + j * kDwBK + (tid + NT * i) / XCH;
            tx[i] = a.perm[p < p1 ? p : p0];
        }
    };
    auto stage_ptr = [&](auto st) -> char* { return decltype(st)::value == 0 ? lds_a : lds_b; };
    auto dma = [&](auto st) {                  // the rows fetch_tokens last fetched
        char* S = stage_ptr(st);
#pragma unroll
        for (int i = 0; i < Q_PER_T; ++i)
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(a.dY + (int64_t)tq[i] * a.ldy + q_off[i]),
                                             (__attribute__((address_space(3))) void*)(S + (NT * i + 64 * wave) * 16), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < X_PER_T; ++i)
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(a.X + (int64_t)tx[i] * a.D + x_off[i]),
                                             (__attribute__((address_space(3))) void*)(S + Q_BYTES + (NT * i + 64 * wave) * 16), 16, 0, 0);
    };
    // Last step: zero the dQ rows past the split (after the barrier that
    // published the stage; ends with a barrier).
    auto fix_tail = [&](int j, auto st) {
        const int valid = p1 - (p0 + j * kDwBK);
        if (valid >= kDwBK) return;            // uniform
        char* S = stage_ptr(st);
        for (int u = tid; u < kDwBK * QCH; u += NT)
            if (u / QCH >= valid) *reinterpret_cast<u32x4*>(S + u * 16) = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto step = [&](int j, auto st) __attribute__((always_inline)) {
        constexpr int SI = decltype(st)::value;
        fix_tail(j, st);
        if (j + 1 < n_steps) {
            dma(StageC<SI ^ 1>{});
            if (j + 2 < n_steps) fetch_tokens(j + 2);
        }
        const char* Qs = stage_ptr(st);
        const char* Xs = Qs + Q_BYTES;
#pragma unroll
        for (int ks = 0; ks < kDwBK / 32; ++ks) {
            Frag<bf16> qf[FM], xf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) qf[i] = ld_frag_tr<QCH>(Qs, 32 * ks, 16 * i, lane);
#pragma unroll
            for (int jn = 0; jn < FN; ++jn) xf[jn] = ld_frag_tr<XCH>(Xs, 32 * ks, 64 * wave + 16 * jn, lane);
            // x fragment as A: the lane ends with 4 consecutive columns of one d row
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int jn = 0; jn < FN; ++jn) acc[i][jn] = mma16(xf[jn], qf[i], acc[i][jn]);
        }
        __syncthreads();    // releases this stage and (waiting for the loads) publishes the next
    };
    if (n_steps > 0) {
        fetch_tokens(0);
        dma(StageC<0>{});
        if (n_steps > 1) fetch_tokens(1);
        __syncthreads();
        for (int j = 0; j < n_steps; j += 2) {
            step(j, StageC<0>{});
            if (j + 1 < n_steps) step(j + 1, StageC<1>{});
        }
    }
    // lane holds dWq row e*D + 16i + l16, columns c0 + 64*wave + 16*jn + 4*(lane/16) .. +3
    float* out = a.part + (int64_t)s * a.split_stride;
    const int l16 = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) {
        const int c = c0 + 64 * wave + 16 * jn + 4 * q4;
        if (c >= a.D) continue;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            *reinterpret_cast<f32x4*>(out + (int64_t)(e * D + 16 * i + l16) * a.D + c) = acc[i][jn];
    }
}

}  // namespace gqe
