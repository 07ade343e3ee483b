// Causal flash attention over dense per-group K/V for many query heads.
//
// The GQE layer runs one attention per picked expert and one for the shared
// head ("Grouped Query Experts" explainer, technical summary, "Architecture
// and routing": every picked expert and the always-on shared head attend over
// their group's unchanged K/V; FrontiersMind GQE article, part 4). The dense
// GQA baseline runs one per query head. Both are the same kernel: a head is a
// query source (base, row stride), a KV group and an output column.
//
// Work split: one workgroup = one KV group, one sequence, NW waves x QW query
// rows, where the rows are all query heads reading that group (for GQE: the
// group's k routed experts, plus the shared head on its group), token by
// token. K/V tiles are staged in double-buffered LDS once and serve every
// head of the group. At head width 64 the softmax's vector work per score is as large as
// the matrix work, so the kernel moves what it can onto the matrix cores:
//   * scores are computed transposed, S^T = K Q^T, so after the softmax every
//     lane already holds the key slots the product O^T = V^T P^T wants as its
//     B operand (no shuffles between the two products);
//   * queries arrive pre-scaled by log2(e)/sqrt(d) (fused into the projection
//     epilogue), and the score accumulator starts at -m (the running max), so
//     p = exp2(S) needs no per-score arithmetic before v_exp_f32;
//   * the softmax denominator is one more MFMA against a row of ones, so it
//     sums exactly the bf16 P used in the numerator;
//   * the running max only moves when a tile exceeds it by more than 8 (log2
//     units); otherwise P may reach 2^8 and nothing is rescaled. Numerator
//     and denominator share the reference, so the result is unchanged;
//   * row maxima reduce across the four lanes of a query with the gfx950
//     permlane swaps (VALU, not LDS).
// V is kept transposed in HBM ([group][d][token]) so its A operand reads
// contiguous keys.
#pragma once

#include "gqe_common.hpp"

namespace gqe {

struct AttnArgs {
    const void* Q0;      // main heads: query of token n, main head j at Q0 + n*q0_ld + j*d
    const void* Q1;      // extra (shared) head: Q1 + n*q1_ld, or null
    const void* K;       // [G][Bt][Tpad][d]
    const void* Vt;      // [G][d][Bt*Tpad]
    void* O;             // main head j -> O + n*o_ld + j*d; extra head -> O + n*o_ld + o1_col
    int64_t q0_ld, q1_ld, o_ld;
    int64_t T, Tpad;
    int32_t Bt;
    int32_t G;           // KV groups
    int32_t R;           // main heads per group: main head j = g*R + r reads group g
    int32_t kv1;         // the group whose rows also carry the extra head (if Q1)
    int32_t n_o;         // row tiles per sequence of a regular group (R rows per token)
    int32_t n_x;         // row tiles per sequence of group kv1 when it carries the extra head
    int32_t o1_col;
    // Optional (training forward): minus the log2-domain log-sum-exp of every
    // row, lse[row_base(g, b) + row] = -log2(sum_k exp2(s_k)) with row = t*Rg
    // + r, where a sequence of a regular group spans lse_Lr rows and one of
    // group kv1 (extra head) lse_Lx. Negated so that the backward's score
    // products can start from it as their accumulator.
    float* lse;
    int64_t lse_Lr, lse_Lx;
};

// First LSE row of group g, sequence b: groups in order, each sequence of a
// regular group lse_Lr rows, of the extra head's group lse_Lx rows.
__device__ __forceinline__ int64_t attn_lse_base(const AttnArgs& a, int g, int b) {
    const bool xg = a.Q1 != nullptr && g == a.kv1;
    const int64_t before = (int64_t)a.Bt * ((int64_t)g * a.lse_Lr + ((a.Q1 != nullptr && g > a.kv1) ? a.lse_Lx - a.lse_Lr : 0));
    return before + (int64_t)b * (xg ? a.lse_Lx : a.lse_Lr);
}

// Tile shapes: queries per wave, waves per workgroup, keys per tile and the
// waves per SIMD the register budget is sized for.
//   * Short sequences: four-wave workgroups of 128 query rows with 64-key
//     tiles (32 KB of LDS for the two stages), three workgroups per CU. The
//     waves that share a SIMD then belong to different workgroups, whose
//     barriers are independent, so one wave's softmax runs while another's
//     products do; with two waves of one eight-wave workgroup per SIMD both
//     met every barrier together and took turns (measured 9% slower at
//     T = 32K, 7% at the k = 2 workload).
//   * Long sequences: eight-wave workgroups of 256 rows with 128-key tiles,
//     one per CU. A query tile reads every K/V tile up to its diagonal, rows
//     x 4d flops for 4d bytes, so once a group's K/V stream outgrows the
//     caches (T = 1M: 256 MB per group) 128-row tiles are held near
//     128 flop/byte x 8 TB/s = 1 PFLOP/s by HBM; 256-row tiles halve those
//     reads (T = 1M: 1.10 s against 1.48 s per layer).
template <int QW_, int NW_, int BKV_, int WPE_>
struct AttnShape {
    static constexpr int QW = QW_, NW = NW_, BKV = BKV_, WPE = WPE_, BQ = NW_ * QW_;
};
#ifndef GQE_ATTN_SHORT_SHAPE
#define GQE_ATTN_SHORT_SHAPE 32, 4, 64, 3
#endif
using AttnShort = AttnShape<GQE_ATTN_SHORT_SHAPE>;
using AttnLong = AttnShape<32, 8, 128, 2>;
// fp32 layers: the short tile with registers for two waves per SIMD (fp32
// fragments are twice the registers; at d = 64 three would not fit).
using AttnShortF32 = AttnShape<32, 4, 64, 2>;
constexpr float kLazyRescale = 8.f;   // log2 units the running max may lag by

// Maximum that propagates NaN (IEEE maximum): gfx950 has it as v_maximum3_f32
// and needs no quieting of the inputs, unlike fmaxf. Scores are never NaN.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max over the four lanes {l16, l16+16, l16+32, l16+48} that hold one query.
__device__ __forceinline__ float quad_row_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Key held by row i of 16-row score block kb. The order makes the eight P
// values a lane holds for one 32-key step eight consecutive keys, so each V^T
// fragment of the second product is one 16-byte LDS read.
__device__ __forceinline__ int key_of_row(int kb, int i) {
    return 32 * (kb >> 1) + 8 * (i >> 2) + 4 * (kb & 1) + (i & 3);
}
// LDS layouts, both measured free of bank conflicts on gfx950 for the reads
// below. K: rows of KCH 16-byte chunks, chunk c of row r at c ^ swz(r), where
// swz spreads the rows key_of_row visits for one block. V^T: rows of VCH
// chunks, chunk c of row r at c ^ (r % VCH).
template <int KCH>
__device__ __forceinline__ int k_chunk_off(int r, int c) {
    const int swz = ((r & 3) | (((r >> 3) & 1) << 2)) & (KCH - 1);
    return r * KCH * 16 + ((c ^ swz) * 16);
}
template <int VCH>
__device__ __forceinline__ int v_chunk_off(int r, int c) {
    return r * VCH * 16 + ((c ^ (r & (VCH - 1))) * 16);
}

// Placement of the units of one level on the XCDs. Workgroup i runs on XCD
// i % 8, so slot p of a level whose first workgroup index is c0 runs on XCD
// (c0 + p) % 8. Regular stream r (a KV group of one sequence, one unit per
// level) has home XCD r % 8: slot p on XCD x that is the k-th slot of the
// level on x takes stream x + 8k when it exists. The other slots take, in
// order, the level's extra units (index nrb + i) and then the regular streams
// that found no home slot. A bijection of [0, c) for any c >= nrb.
__device__ __forceinline__ int64_t level_slot_unit(int64_t p, int64_t c, int s0, int64_t nrb) {
    auto visits = [&](int x, int64_t upto) -> int64_t {   // slots before upto on XCD x
        const int d = (x - s0) & 7;
        return upto > d ? (upto - d - 1) / 8 + 1 : 0;
    };
    auto homes = [&](int x) -> int64_t { return nrb > x ? (nrb - 1 - x) / 8 + 1 : 0; };
    const int x = (int)((s0 + p) & 7);
    const int64_t k = visits(x, p);
    if (k < homes(x)) return x + 8 * k;
    int64_t rank = p;                                     // overflow slots before p
    for (int y = 0; y < 8; ++y) rank -= min(visits(y, p), homes(y));
    const int64_t nx = c - nrb;
    if (rank < nx) return nrb + rank;
    int64_t left = rank - nx;
    for (int y = 0; y < 8; ++y) {
        const int64_t lo = visits(y, c), hi = homes(y);
        if (hi > lo) {
            if (left < hi - lo) return y + 8 * (lo + left);
            left -= hi - lo;
        }
    }
    return 0;   // not reached for p < c
}

template <int N>
struct StageC {
    static constexpr int value = N;
};

template <typename T, int D, class Shape>
__global__ __launch_bounds__(Shape::NW * 64) __attribute__((amdgpu_waves_per_eu(Shape::WPE, Shape::WPE)))
void attn_fwd_kernel(AttnArgs a) {
    constexpr int NW = Shape::NW, QW = Shape::QW;
    constexpr int NT = NW * 64;
    constexpr int QB = QW / 16;           // 16-query blocks per wave
    constexpr int BQ = Shape::BQ;
    constexpr int BKV = Shape::BKV;
    constexpr int KB = BKV / 16;               // 16-key blocks per tile
    constexpr int KC = BKV / 32;               // 32-key steps of the second product
    constexpr int ES = sizeof(T);
    constexpr int DK = D / 32;                 // 32-wide contraction steps over d
    constexpr int CB = D / 16;                 // 16-wide blocks of the output columns
    constexpr int KCH = D * ES / 16;           // 16-byte chunks per K row
    constexpr int VCH = BKV * ES / 16;         // 16-byte chunks per V^T row
    constexpr int K_BYTES = BKV * KCH * 16, V_BYTES = D * VCH * 16;
    constexpr int STAGE = K_BYTES + V_BYTES;
    constexpr int K_PER_T = BKV * KCH / NT;    // 16-byte chunks each thread stages per tile
    constexpr int V_PER_T = D * VCH / NT;
    static_assert(BKV * KCH % NT == 0 && D * VCH % NT == 0, "a tile splits evenly over the threads");
    constexpr int VEC = 16 / ES;
    // Two LDS stages as separate arrays: the compiler can then tell reads of
    // one stage from the direct global->LDS loads filling the other.
    __shared__ __attribute__((aligned(16))) char lds_a[STAGE];
    __shared__ __attribute__((aligned(16))) char lds_b[STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    // The wave index is uniform across the wave; saying so keeps everything
    // derived from it (row ranges, skip and mask tests) in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    // Work unit: one KV group of one sequence and one tile of BQ query rows.
    // A group's rows are its R main heads token by token (row = t*Rg + r),
    // plus the extra head for group kv1, so one staged K/V tile serves every
    // query head that reads this group. Groups thus come in two classes:
    // regular (R rows per token, n_o tiles) and the extra group (R+1 rows per
    // token, n_x tiles). Workgroups are ordered by level, longest rows first:
    // level l holds tile n_o-1-l of every regular group and the extra group's
    // tiles that end at about the same token, [n_x - e(l+1), n_x - e(l)) with
    // e(l) = l*n_x/n_o; count(l) workgroups precede level l. Inside a level
    // the units are placed by level_slot_unit so that each regular stream
    // stays on one XCD (and one L2) from level to level.
    const bool xcls = a.Q1 != nullptr;
    const int n_reg = xcls ? a.G - 1 : a.G;                // regular groups
    const int64_t nrb = (int64_t)a.Bt * n_reg;              // regular workgroups per level
    auto count = [&](int l) -> int64_t {
        return nrb * l + (xcls ? (int64_t)a.Bt * ((int64_t)l * a.n_x / a.n_o) : 0);
    };
    const int64_t L = blockIdx.x;
    int lv = (int)((double)L / ((double)nrb + (xcls ? (double)a.Bt * a.n_x / a.n_o : 0.0)));
    lv = min(max(lv, 0), a.n_o - 1);
    while (lv > 0 && count(lv) > L) --lv;
    while (lv + 1 < a.n_o && count(lv + 1) <= L) ++lv;
    const int64_t c0 = count(lv);
    const int64_t pos = level_slot_unit(L - c0, count(lv + 1) - c0, (int)(c0 & 7), nrb);
    int g, b, qt, Rg;
    if (pos < nrb) {
        const int gi = (int)(pos / a.Bt);
        b = (int)(pos % a.Bt);
        g = (xcls && gi >= a.kv1) ? gi + 1 : gi;
        qt = a.n_o - 1 - lv;
        Rg = a.R;
    } else {
        const int64_t q = pos - nrb;
        b = (int)(q % a.Bt);
        g = a.kv1;
        qt = a.n_x - 1 - (int)((int64_t)lv * a.n_x / a.n_o) - (int)(q / a.Bt);
        Rg = a.R + 1;
    }
    const int64_t T_ = a.T;
    const int64_t n_rows = T_ * Rg;
    const T* Kg = (const T*)a.K + ((int64_t)g * a.Bt + b) * a.Tpad * D;
    const int64_t vrow = (int64_t)a.Bt * a.Tpad;
    const T* Vg = (const T*)a.Vt + (int64_t)g * D * vrow + (int64_t)b * a.Tpad;
    const int64_t tok0 = (int64_t)b * T_;
    const int row0 = qt * BQ + wave * QW;           // first row of this wave
    // Token of each row this lane holds (query column l16 of block qb).
    int tq[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) tq[qb] = (row0 + qb * 16 + l16) / Rg;
    const int t_first = row0 / Rg;                       // tokens spanned by this wave
    const int t_last = (int)min<int64_t>(T_ - 1, (row0 + QW - 1) / Rg);
    // Query and output row pointers of a row (token t, head slot r).
    auto q_row = [&](int t, int r) -> const T* {
        return r < a.R ? (const T*)a.Q0 + (tok0 + t) * a.q0_ld + (int64_t)(g * a.R + r) * D
                       : (const T*)a.Q1 + (tok0 + t) * a.q1_ld;
    };
    auto o_row = [&](int t, int r) -> T* {
        return (T*)a.O + (tok0 + t) * a.o_ld + (r < a.R ? (int64_t)(g * a.R + r) * D : (int64_t)a.o1_col);
    };

    // Queries (pre-scaled) as the B operand of S^T = K Q^T.
    Frag<T> qf[QB][DK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int rho = row0 + qb * 16 + l16;
        const T* qp = (rho < n_rows) ? q_row(tq[qb], rho % Rg) : nullptr;
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            if (qp != nullptr) {
                qf[qb][dk] = ld_frag<T>(qp + dk * 32 + 8 * q4);
            } else {
                if constexpr (ES == 2) {
                    qf[qb][dk].v = bf16x8{};
                } else {
                    qf[qb][dk].lo = f32x4{0.f, 0.f, 0.f, 0.f};
                    qf[qb][dk].hi = qf[qb][dk].lo;
                }
            }
        }
    }
    // A operand of the denominator product: row 0 of the block is all ones.
    Frag<T> ones;
    {
        const float o1 = (l16 == 0) ? 1.f : 0.f;
        if constexpr (ES == 2) {
#pragma unroll
            for (int i = 0; i < 8; ++i) ones.v[i] = (bf16)o1;
        } else {
            ones.lo = f32x4{o1, o1, o1, o1};
            ones.hi = ones.lo;
        }
    }

    f32x4 o[CB][QB], lsum[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        lsum[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) o[cb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Reference m subtracted from the scores of each query (log2 units),
    // kept as the C operand that starts every score block (-m, or 0 until the
    // first tile sets it) and as the rebase threshold (-inf until set, then
    // kLazyRescale): both change only when the reference moves.
    f32x4 minit[QB];
    float thr[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        minit[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        thr[qb] = -INFINITY;
    }

    // Keys up to the last token of the tile.
    const int t_hi = (int)min<int64_t>(T_ - 1, ((int64_t)qt * BQ + BQ - 1) / Rg);
    const int n_kv = t_hi / BKV + 1;

    // Tiles are staged with gfx950's direct global->LDS loads: one
    // instruction moves 16 bytes per lane into 64 consecutive 16-byte LDS
    // slots of the wave, so each lane loads the global chunk that the
    // swizzled layout puts in its slot (slot p of row r holds chunk
    // p ^ swz(r)). Offsets relative to the tile's first key are fixed per
    // thread. Keys at or beyond T: K rows there are masked off by the causal
    // test; V^T columns there are zeroed in LDS before use (fix_tail).
    int koff[K_PER_T];
    int64_t voff[V_PER_T];
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
        const int it = tid + NT * i, r = it / KCH, p = it % KCH;
        koff[i] = r * D + (p ^ (((r & 3) | (((r >> 3) & 1) << 2)) & (KCH - 1))) * VEC;
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
        const int it = tid + NT * i, r = it / VCH, p = it % VCH;
        voff[i] = (int64_t)r * vrow + (int64_t)(p ^ (r & (VCH - 1))) * VEC;
    }
    auto stage_ptr = [&](auto stage) -> char* { return decltype(stage)::value == 0 ? lds_a : lds_b; };
    auto dma = [&](int j, auto stage) {
        const int64_t s0 = (int64_t)j * BKV;
        char* Ks = stage_ptr(stage);
        char* Vs = Ks + K_BYTES;
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i)
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(Kg + s0 * D + koff[i]),
                                             (__attribute__((address_space(3))) void*)(Ks + (NT * i + 64 * wave) * 16),
                                             16, 0, 0);
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i)
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(Vg + s0 + voff[i]),
                                             (__attribute__((address_space(3))) void*)(Vs + (NT * i + 64 * wave) * 16),
                                             16, 0, 0);
    };
    // Last tile of a sequence: zero the V^T entries of keys >= T (their P is
    // 0, but padding may hold anything). Call after the tile's barrier; ends
    // with a barrier.
    auto fix_tail = [&](int j, auto stage) {
        const int s0 = j * BKV;
        if (s0 + BKV <= T_) return;                     // uniform
        char* Vs = stage_ptr(stage) + K_BYTES;
        for (int it = tid; it < D * VCH; it += NT) {
            const int r = it / VCH, c = it % VCH, k0 = s0 + c * VEC;
            if (k0 + VEC <= T_) continue;
            T* e = reinterpret_cast<T*>(Vs + v_chunk_off<VCH>(r, c));
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                if (k0 + q >= T_) e[q] = from_f32<T>(0.f);
        }
        __syncthreads();
    };

    // One key tile; the LDS stage is a compile-time constant so every LDS
    // address is a per-lane base plus an immediate offset.
    auto tile = [&](int j, auto stage) {
        constexpr int ST = decltype(stage)::value;
        fix_tail(j, stage);
        if (j + 1 < n_kv) dma(j + 1, StageC<ST ^ 1>{});
        const int s0 = j * BKV;
        if (s0 <= t_last) {                    // else every key is above every query of this wave
            const char* Ks = stage_ptr(stage);
            const char* Vs = Ks + K_BYTES;
            // S^T = K Q^T - m, accumulated from the current reference.
            // The first MFMA of every block takes -m as its C operand.
            f32x4 s[KB][QB];
#pragma unroll
            for (int dk = 0; dk < DK; ++dk)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const int kr = key_of_row(kb, l16), kc0 = (dk * 32 + 8 * q4) * ES / 16;
                    Frag<T> kf;
                    if constexpr (ES == 2) {
                        kf = ld_frag<T>(Ks + k_chunk_off<KCH>(kr, kc0));
                    } else {   // 32 bytes = two swizzled chunks
                        kf.lo = *reinterpret_cast<const f32x4*>(Ks + k_chunk_off<KCH>(kr, kc0));
                        kf.hi = *reinterpret_cast<const f32x4*>(Ks + k_chunk_off<KCH>(kr, kc0 + 1));
                    }
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mma16(kf, qf[qb][dk], dk == 0 ? minit[qb] : s[kb][qb]);
                }
            if (s0 + BKV - 1 > t_first) {      // a key may lie above a query: causal mask
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int key = s0 + key_of_row(kb, 4 * q4 + v);
                            if (key > tq[qb]) s[kb][qb][v] = -INFINITY;
                        }
            }
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mx = s[0][qb][0];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) mx = vmax(mx, s[kb][qb][v]);
                // Move the reference only when needed: first tile, or scores
                // more than kLazyRescale above it. A column passes the
                // threshold exactly when one of its four lanes' shares does, so
                // the shares decide first and the column maximum is formed only
                // when some column moves.
                if (__builtin_amdgcn_ballot_w64(mx > thr[qb]) != 0) {
                    mx = quad_row_max(mx);
                    const bool need = mx > thr[qb];
                    const float delta = need ? mx : 0.f;
                    const float corr = __builtin_amdgcn_exp2f(-delta);
                    minit[qb] -= delta;
                    thr[qb] = need ? kLazyRescale : thr[qb];
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) s[kb][qb] -= delta;
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) o[cb][qb] *= corr;
                    lsum[qb] *= corr;
                }
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) s[kb][qb][v] = __builtin_amdgcn_exp2f(s[kb][qb][v]);
            }
            // O^T += V^T P^T and l += 1^T P^T, 32 keys per step: slot jj of lane
            // group q4 is key 32*kc + 8*q4 + jj (blocks 2kc and 2kc+1, see key_of_row).
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                Frag<T> pf[QB];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    if constexpr (ES == 2) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            pf[qb].v[v] = (bf16)s[2 * kc][qb][v];
                            pf[qb].v[4 + v] = (bf16)s[2 * kc + 1][qb][v];
                        }
                    } else {
                        pf[qb].lo = s[2 * kc][qb];
                        pf[qb].hi = s[2 * kc + 1][qb];
                    }
                    lsum[qb] = mma16(ones, pf[qb], lsum[qb]);
                }
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    // Keys 32*kc + 8*q4 .. +7 of V^T row cb*16 + l16.
                    const int vr = cb * 16 + l16, vc = (32 * kc + 8 * q4) * ES / 16;
                    Frag<T> vf;
                    if constexpr (ES == 2) {
                        vf = ld_frag<T>(Vs + v_chunk_off<VCH>(vr, vc));
                    } else {
                        vf.lo = *reinterpret_cast<const f32x4*>(Vs + v_chunk_off<VCH>(vr, vc));
                        vf.hi = *reinterpret_cast<const f32x4*>(Vs + v_chunk_off<VCH>(vr, vc + 1));
                    }
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) o[cb][qb] = mma16(vf, pf[qb], o[cb][qb]);
                }
            }
        }
        __syncthreads();    // releases this stage and (waiting for the loads) publishes the next
    };

    dma(0, StageC<0>{});
    __syncthreads();
    for (int j = 0; j < n_kv; j += 2) {
        tile(j, StageC<0>{});
        if (j + 1 < n_kv) tile(j + 1, StageC<1>{});
    }

    // Normalise and store. The denominator sits in row 0 of lsum (lanes of
    // lane group 0, element 0); lane holds query l16 of block qb, columns
    // cb*16 + 4*q4 + v.
    const int64_t lse0 = a.lse != nullptr ? attn_lse_base(a, g, b) : 0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = __shfl(lsum[qb][0], l16);
        const float inv = 1.f / l;
        const int rho = row0 + qb * 16 + l16;
        if (rho >= n_rows) continue;
        // p = exp2(s - m) / l, so log2 of the normaliser is m + log2(l), m = -minit.
        if (a.lse != nullptr && q4 == 0) a.lse[lse0 + rho] = minit[qb][0] - __builtin_amdgcn_logf(l);
        T* orow = o_row(tq[qb], rho % Rg);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            T* op = orow + cb * 16 + 4 * q4;
            if constexpr (ES == 2) {
                bf16x4 w;
#pragma unroll
                for (int v = 0; v < 4; ++v) w[v] = (bf16)(o[cb][qb][v] * inv);
                *reinterpret_cast<bf16x4*>(op) = w;
            } else {
                f32x4 w;
#pragma unroll
                for (int v = 0; v < 4; ++v) w[v] = o[cb][qb][v] * inv;
                *reinterpret_cast<f32x4*>(op) = w;
            }
        }
    }
}

}  // namespace gqe
