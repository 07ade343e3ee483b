// One decode step of the GQE layer over a dense KV cache: one new token per
// sequence. The K/V projections and the cache are those of the underlying
// GQA model, unchanged; only the query side is sparse ("Grouped Query
// Experts" explainer, technical summary, "Architecture and routing";
// FrontiersMind GQE article, part 4). Reading the cache dominates, so the
// attention kernel is an HBM stream:
//   * the token projections (K, V, shared query, router logits) by
//     skinny_proj_kernel, one pass over the weights;
//   * decode_token_kernel: per (sequence, group, rank, 16 query columns), the
//     group's routing and the picked expert's query; it also appends the new
//     key row and value column to the cache;
//   * attn_decode_kernel: one workgroup per (sequence, group, chunk of cached
//     keys); each wave streams its keys straight from HBM into MFMA operands
//     (K rows as the A operand of S^T = K Q^T, V^T rows as the A operand of
//     O^T = V^T P^T) for all query heads of the group at once (the picked
//     experts and, on its group, the shared head, zero-padded to 16), with an
//     online softmax, and writes the chunk's (max, sum, unnormalised output);
//   * decode_combine_kernel: per sequence, merges the chunks of every head
//     into its slot of C = [hard | weighted | shared] and then forms the
//     weighted slot from the hard ones, for the output projection, again a
//     skinny_proj_kernel pass.
// The cache layout is the prefill's: keys [G][B][T][d] (one contiguous row
// per key), values transposed [G][d][B*T] (contiguous keys per column).
#pragma once

#include "attention.hpp"
#include "gemm.hpp"
#include "route.hpp"

namespace gqe {

// Token side, one workgroup per (sequence b, group g, rank r, block cb of 16
// query columns): the group's top-k from the router logits (as route_kernel
// picks them), then columns 16cb .. 16cb+15 of the picked expert's query
// Qr[b][g*k + r] = x[b] Wq_e^T (pre-scaled), one pass over those Wq rows as in
// skinny_proj_kernel (every product column is token b; lanes of column 0
// store). Workgroups with r = 0 and cb = 0 also append the new key row and
// value column at pos[b]; workgroup (b, 0, 0, 0) writes the token's full
// routing (idx, renormalised w).
struct DecTokArgs {
    const float* logits;  // [B, G*M]
    const bf16* x;        // [B, D]
    const bf16* Wq;       // [G*M*d, D]
    const bf16* Kn;       // [B, G*d] the new keys
    const bf16* Vn;       //          and values
    const int32_t* pos;
    int32_t* idx;         // [B, G*k]
    float* w;
    bf16* Qr;             // [B, G*k, d]
    bf16* kc;             // [G][B][T][d]
    bf16* vtc;            // [G][d][B*T]
    int64_t T, D;
    int32_t Bt, G, M, k, d;
    float qscale;
};

template <int MM>   // as in route_kernel
__global__ __launch_bounds__(256) void decode_token_kernel(DecTokArgs a) {
    __shared__ int32_t s_sel[256];   // token b's picks [g*k + r] (G*k <= 256)
    __shared__ float s_p[256];       // and their probabilities within the group
    __shared__ float s_inv;
    __shared__ f32x4 part[3][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    const int ncb = a.d / 16;
    int u = blockIdx.x;
    const int cb = u % ncb;
    u /= ncb;
    const int r = u % a.k;
    u /= a.k;
    const int g = u % a.G, b = u / a.G;
    const float* z = a.logits + (int64_t)b * a.G * a.M;
    // Every group's top-k, one thread per group.
    for (int gg = tid; gg < a.G; gg += 256)
        topk_group<MM>(z + gg * a.M, a.M, a.k, [&](int rr, int m, float pr) {
            s_sel[gg * a.k + rr] = m;
            s_p[gg * a.k + rr] = pr;
        });
    __syncthreads();
    if (g == 0 && r == 0 && cb == 0) {
        // The token's routing as route_kernel writes it: the same picks, and
        // the probabilities renormalised by the same sum (renorm_total).
        const int GK = a.G * a.k;
        if (tid == 0) s_inv = 1.f / renorm_total(a.G, a.k, [&](int gg, int rr) { return s_p[gg * a.k + rr]; });
        __syncthreads();
        for (int q = tid; q < GK; q += 256) {
            a.idx[(int64_t)b * GK + q] = s_sel[q];
            a.w[(int64_t)b * GK + q] = s_p[q] * s_inv;
        }
    }
    const int64_t p = a.pos[b];
    if (r == 0 && cb == 0 && tid < a.d && p >= 0 && p < a.T) {
        const int64_t src = ((int64_t)b * a.G + g) * a.d + tid;
        a.kc[(((int64_t)g * a.Bt + b) * a.T + p) * a.d + tid] = a.Kn[src];
        a.vtc[((int64_t)g * a.d + tid) * ((int64_t)a.Bt * a.T) + (int64_t)b * a.T + p] = a.Vn[src];
    }
    const int e = g * a.M + s_sel[g * a.k + r];
    const bf16* wrow = a.Wq + ((int64_t)e * a.d + cb * 16 + l16) * a.D;
    f32x4 acc = skinny_dot(wrow, a.x + (int64_t)b * a.D, (int)a.D, wave, q4);
    if (!skinny_reduce(acc, part, wave, lane) || l16 != 0) return;
    bf16x4 q;
#pragma unroll
    for (int v = 0; v < 4; ++v) q[v] = (bf16)(acc[v] * a.qscale);
    *reinterpret_cast<bf16x4*>(a.Qr + (((int64_t)b * a.G + g) * a.k + r) * a.d + cb * 16 + 4 * q4) = q;
}

struct DecodeArgs {
    const bf16* Qr;       // [B, G*k, d] routed queries (pre-scaled by log2(e)/sqrt(d))
    const bf16* Qsh;      // [B, d] shared-head query (pre-scaled)
    const bf16* K;        // [G][B][T][d]
    const bf16* Vt;       // [G][d][B*T]
    const int32_t* pos;   // [B]: the new token sits at pos[b]; keys 0 .. pos[b] are attended
    float* part_o;        // [B][G][n_ch][R16][d] unnormalised outputs (relative to part_m)
    float* part_ml;       // [B][G][n_ch][R16][2] (max, sum) in log2 units
    int64_t T;
    int32_t Bt, G, k, s0, d;
    int32_t n_ch;         // chunks per sequence
    int32_t R16;          // head slots per group, a multiple of 16 (>= k + 1)
};

#ifndef GQE_DEC_WPE
#define GQE_DEC_WPE 2
#endif
#ifndef GQE_DEC_LINES
#define GQE_DEC_LINES 1
#endif

// Key (within a 64-key step) of row i of score block kb when K is read in
// whole lines: block pairs (2h, 2h + 1) give product step h its keys
// 16*q4 + 8*h + e, matching the V^T fragments lines_to_frags builds.
__device__ __forceinline__ int dec_key(int kb, int i) {
    return 16 * (i >> 2) + 8 * (kb >> 1) + 4 * (kb & 1) + (i & 3);
}

// Two whole-line loads of 16 rows (a: rows 0-7, b: rows 8-15; lane (l16, q4)
// holds row l16 & 7 of its half, 16-byte chunk (l16 >> 3) + 2*q4) become two
// MFMA fragments: lane (l16, q4) of a / b then holds row l16, chunk 2*q4 / 2*q4 + 1.
// Lanes l16 and l16 ^ 8 trade one register's worth: a row rotation by 8 lanes
// written to half of each row's lanes.
__device__ __forceinline__ void lines_to_frags(u32x4& a, u32x4& b) {
    u32x4 f0, f1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f0[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)a[i], (int)b[i], 0x128, 0xF, 0xC, false);
        f1[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)b[i], (int)a[i], 0x128, 0xF, 0x3, false);
    }
    a = f0;
    b = f1;
}

__device__ __forceinline__ Frag<bf16> as_frag(u32x4 u) {
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8, u);
    return f;
}

// A raw buffer view of n bytes at p (p uniform over the wave).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

// A 16-byte streaming buffer load at byte offset off (per lane): the cache is
// read once, so its lines need not stay in L2. Offsets at or past the view's
// size read as zeros (the whole offset is the lane's, so the check sees it).
__device__ __forceinline__ u32x4 ld16_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
constexpr int kDecNW = 4;          // waves per workgroup

// CW keys per wave, kDecNW * CW per chunk (workgroup).
template <int D, int CW>
__global__ __launch_bounds__(kDecNW * 64) __attribute__((amdgpu_waves_per_eu(GQE_DEC_WPE)))
void attn_decode_kernel(DecodeArgs a) {
    constexpr int DK = D / 32, CB = D / 16;
    constexpr int KS = 64;                          // keys per step
    constexpr int KB = KS / 16, KH = KS / 32;       // 16-key score blocks, 32-key product steps
    constexpr int NB = CW / KS;                     // steps per wave
    constexpr bool kLines = GQE_DEC_LINES && D % 64 == 0;
    // Key of row i of score block kb (rows 4*q4 + v of a lane's result).
    auto row_key = [](int kb, int i) { return kLines ? dec_key(kb, i) : key_of_row(kb, i); };
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    const int ch = blockIdx.x % a.n_ch;
    const int bg = blockIdx.x / a.n_ch, g = bg % a.G, b = bg / a.G;
    const int64_t p = a.pos[b];
    if (p < 0 || p >= a.T) return;                  // not a cache position: nothing is read
    const int64_t len = p + 1;                      // keys 0 .. pos[b]
    const int64_t c0 = (int64_t)ch * (kDecNW * CW);
    if (c0 >= len) return;                          // the combine reads chunks below len only
    const int Rg = a.k + (g == a.s0 ? 1 : 0);
    const bf16* Kg = a.K + ((int64_t)g * a.Bt + b) * a.T * D;
    const int64_t vrow = (int64_t)a.Bt * a.T;
    const bf16* Vg = a.Vt + (int64_t)g * D * vrow + (int64_t)b * a.T;
    // Buffer views (sizes below 4 GiB by the host's checks): this sequence's
    // K rows, and V^T from its first column to the end of its last row.
    const __amdgpu_buffer_rsrc_t rsK = make_rsrc(Kg, (uint32_t)(a.T * 2 * D));
    const __amdgpu_buffer_rsrc_t rsV = make_rsrc(Vg, (uint32_t)(((int64_t)(D - 1) * vrow + a.T) * 2));
    const uint32_t kvoff = (uint32_t)((16 * ((l16 >> 2) & 1) + (l16 & 3)) * (2 * D) + 16 * ((l16 >> 3) + 2 * q4));
    const uint32_t vvoff = (uint32_t)((l16 & 7) * vrow * 2 + 16 * ((l16 >> 3) + 2 * q4));

    __shared__ float s_m[kDecNW][16], s_l[kDecNW][16];
    __shared__ float s_o[kDecNW][D][16];

    for (int h0 = 0; h0 < Rg; h0 += 16) {           // 16 heads per pass (one pass unless k >= 16)
        // Queries as the B operand: column l16 = head h0 + l16 (zero beyond Rg).
        Frag<bf16> qf[DK];
        const int hd = h0 + l16;
        const bf16* qp = hd < a.k ? a.Qr + ((int64_t)b * a.G * a.k + (int64_t)g * a.k + hd) * D
                                  : (hd < Rg ? a.Qsh + (int64_t)b * D : nullptr);
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            if (qp != nullptr) qf[dk] = ld_frag<bf16>(qp + (kLines ? 64 * (dk >> 1) + 16 * q4 + 8 * (dk & 1) : dk * 32 + 8 * q4));
            else qf[dk].v = bf16x8{};
        }
        Frag<bf16> ones;
#pragma unroll
        for (int i = 0; i < 8; ++i) ones.v[i] = (bf16)(l16 == 0 ? 1.f : 0.f);
        f32x4 o[CB], lsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY;                         // running max of head l16 (log2 units)

        const int64_t w0 = c0 + (int64_t)wave * CW;
        const int nb = (int)max<int64_t>(0, min<int64_t>(NB, (len - w0 + KS - 1) / KS));
        // The loads of one step of KS keys: K rows (A of S^T) and V^T rows
        // (A of O^T), KS keys (128 bytes) of each V^T row. With kLines each
        // load instruction reads whole 128-byte lines (8 rows, lane (l16, q4)
        // taking row l16 & 7 of its half and 16-byte chunk (l16 >> 3) + 2*q4)
        // as streaming buffer loads, and lines_to_frags then trades halves
        // between lanes l16 and l16 ^ 8, which leaves chunk 2*q4 + h of row
        // l16 in register h: fragment h's contraction element 8*q4 + e is d
        // (or key) 16*q4 + 8*h + e, on K, Q and V^T alike. Rows past the cache
        // end (the last step when T is not a multiple of KS) lie outside the
        // K buffer and read as zeros; their V^T columns read the next row's
        // first keys (or zeros after the last row). Otherwise (d = 32, whose
        // fragments already cover whole lines of K) each lane loads its
        // fragment directly and keys past the cache end read the last row.
        // Either way those keys lie past len and are masked below.
        auto load = [&](int j, u32x4 (&kl)[KB][DK], u32x4 (&vl)[CB][KH]) {
            const int64_t k0 = w0 + (int64_t)KS * j;
            if constexpr (kLines) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int dk = 0; dk < DK; ++dk) {
                        const int64_t key = k0 + 32 * (dk & 1) + 8 * (kb >> 1) + 4 * (kb & 1);   // + the lane's rows
                        kl[kb][dk] = ld16_buf(rsK, kvoff + (uint32_t)(key * (2 * D) + 128 * (dk >> 1)));
                    }
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int h = 0; h < KH; ++h)
                        vl[cb][h] = ld16_buf(rsV, vvoff + (uint32_t)(((int64_t)(16 * cb + 8 * h) * vrow + k0) * 2));
            } else {
                const bool tail = k0 + KS > a.T;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    int64_t kr = k0 + key_of_row(kb, l16);
                    if (tail) kr = min<int64_t>(kr, a.T - 1);
#pragma unroll
                    for (int dk = 0; dk < DK; ++dk) kl[kb][dk] = ld16(Kg + kr * D + dk * 32 + 8 * q4);
                }
#pragma unroll
                for (int h = 0; h < KH; ++h) {
                    int64_t kc = k0 + 32 * h + 8 * q4;
                    if (tail) kc = min<int64_t>(kc, a.T - 8);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) vl[cb][h] = ld16(Vg + (int64_t)(cb * 16 + l16) * vrow + kc);
                }
            }
        };
        u32x4 kA[KB][DK], vA[CB][KH], kB[KB][DK], vB[CB][KH];
        auto compute = [&](int j, u32x4 (&kl)[KB][DK], u32x4 (&vl)[CB][KH]) {
            const int64_t k0 = w0 + (int64_t)KS * j;
            if constexpr (kLines) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int dk = 0; dk < DK; dk += 2) lines_to_frags(kl[kb][dk], kl[kb][dk + 1]);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) lines_to_frags(vl[cb][0], vl[cb][1]);
            }
            f32x4 s[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dk = 0; dk < DK; ++dk) s[kb] = mma16(as_frag(kl[kb][dk]), qf[dk], s[kb]);
            }
            if (k0 + KS > len) {
                // Keys at or past len are not attended: their scores become -inf
                // and their values 0 (the cache there may hold any bits, and a
                // NaN times a zero probability would still be NaN).
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (k0 + row_key(kb, 4 * q4 + v) >= len) s[kb][v] = -INFINITY;
#pragma unroll
                for (int h = 0; h < KH; ++h)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            // dword i holds keys 2i (low half) and 2i + 1 (high half)
                            const int64_t key = k0 + (kLines ? 16 * q4 + 8 * h : 32 * h + 8 * q4) + 2 * i;
                            if (key >= len) vl[cb][h][i] = 0u;
                            else if (key + 1 >= len) vl[cb][h][i] &= 0xffffu;
                        }
            }
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int v = 0; v < 4; ++v) mx = vmax(mx, s[kb][v]);
            mx = quad_row_max(mx);
            const float mn = vmax(m, mx);
            const float corr = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first step (m = -inf)
            m = mn;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) o[cb] *= corr;
            lsum *= corr;
#pragma unroll
            for (int h = 0; h < KH; ++h) {
                Frag<bf16> pf;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    pf.v[v] = (bf16)__builtin_amdgcn_exp2f(s[2 * h][v] - mn);
                    pf.v[4 + v] = (bf16)__builtin_amdgcn_exp2f(s[2 * h + 1][v] - mn);
                }
                lsum = mma16(ones, pf, lsum);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) o[cb] = mma16(as_frag(vl[cb][h]), pf, o[cb]);
            }
        };
        // Two register sets: the next step's loads are in flight during this step's products.
        if (nb > 0) load(0, kA, vA);
        for (int j = 0; j < nb; j += 2) {
            if (j + 1 < nb) load(j + 1, kB, vB);
            compute(j, kA, vA);
            if (j + 1 < nb) {
                if (j + 2 < nb) load(j + 2, kA, vA);
                compute(j + 1, kB, vB);
            }
        }
        // Merge the waves: lane (l16, q4) holds head l16, columns 16cb + 4*q4 + v.
        const float l = __shfl(lsum[0], l16);
        if (q4 == 0) {
            s_m[wave][l16] = nb > 0 ? m : -INFINITY;
            s_l[wave][l16] = nb > 0 ? l : 0.f;
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int v = 0; v < 4; ++v) s_o[wave][cb * 16 + 4 * q4 + v][l16] = nb > 0 ? o[cb][v] : 0.f;
        __syncthreads();
        const int64_t pbase = (((int64_t)b * a.G + g) * a.n_ch + ch) * a.R16 + h0;
        for (int u = tid; u < 16 * D; u += kDecNW * 64) {
            const int hh = u / D, c = u % D;
            if (h0 + hh >= Rg) continue;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kDecNW; ++w) M = vmax(M, s_m[w][hh]);
            float so = 0.f, sl = 0.f;
#pragma unroll
            for (int w = 0; w < kDecNW; ++w) {
                const float f = s_m[w][hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[w][hh] - M);
                so += f * s_o[w][c][hh];
                sl += f * s_l[w][hh];
            }
            a.part_o[(pbase + hh) * D + c] = so;
            if (c == 0) {
                a.part_ml[(pbase + hh) * 2] = M;
                a.part_ml[(pbase + hh) * 2 + 1] = sl;
            }
        }
        __syncthreads();
    }
}

// Merges the chunks of every head of one sequence (workgroup b; head j =
// g*k + r for routed head r of group g, j = G*k for the shared head) into
// its slot of C[b] = [O_0 .. O_{Gk-1} | weighted | O_sh] in bf16, then forms
// the weighted slot from the bf16 hard slots as the prefill's combine does
// (fp32 sum in slot order). One wave per head at a time (heads wave, wave +
// waves, ...): the lanes read the chunks' (max, sum) pairs 64 at a time,
// then lane c sums column c of the chunks' outputs with eight chunks' loads
// in flight.
constexpr int kDecCombMaxWaves = 16;
__global__ __launch_bounds__(kDecCombMaxWaves * 64) void decode_combine_kernel(
    const float* part_o, const float* part_ml, const float* w, const int32_t* pos, bf16* C, int G, int k, int s0,
    int d, int n_ch, int ch_keys, int R16, int64_t ldc, int64_t T) {
    const int GK = G * k;
    const int b = blockIdx.x, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nw = blockDim.x >> 6;
    const int64_t p = pos[b];
    // An out-of-range position reads no chunk (its slots are unspecified).
    const int64_t len = (p < 0 || p >= T) ? 0 : p + 1;
    const int nch = (int)min<int64_t>(n_ch, (len + ch_keys - 1) / ch_keys);
    if (nch == 0) return;                                         // uniform over the workgroup
    bf16* Cb = C + (int64_t)b * ldc;
    for (int j = wave; j <= GK; j += nw) {
        const int g = j < GK ? j / k : s0, hd = j < GK ? j % k : k;   // the shared head is group s0's row k
        const int64_t hb = (((int64_t)b * G + g) * n_ch) * R16 + hd;
        const float* ml = part_ml + hb * 2;
        const int64_t mls = (int64_t)R16 * 2;
        float M = -INFINITY;
        for (int i = lane; i < nch; i += 64) M = vmax(M, ml[i * mls]);
        for (int o = 32; o > 0; o >>= 1) M = vmax(M, __shfl_xor(M, o));
        float sl = 0.f;
        for (int i = lane; i < nch; i += 64) sl += __builtin_amdgcn_exp2f(ml[i * mls] - M) * ml[i * mls + 1];
        for (int o = 32; o > 0; o >>= 1) sl += __shfl_xor(sl, o);
        if (lane < d) {
            const float* po = part_o + hb * d + lane;
            const int64_t pos_ = (int64_t)R16 * d;
            float so = 0.f;
            int i = 0;
            for (; i + 8 <= nch; i += 8) {
                float f[8], v[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    f[q] = ml[(i + q) * mls];
                    v[q] = po[(i + q) * pos_];
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) so += __builtin_amdgcn_exp2f(f[q] - M) * v[q];
            }
            for (; i < nch; ++i) so += __builtin_amdgcn_exp2f(ml[i * mls] - M) * po[i * pos_];
            Cb[(j < GK ? (int64_t)j : (int64_t)GK + 1) * d + lane] = (bf16)(so / sl);
        }
    }
    __syncthreads();   // the hard slots written above, visible to the whole workgroup
    const float* wb = w + (int64_t)b * GK;
    for (int c = threadIdx.x; c < d; c += blockDim.x) {
        float acc = 0.f;
        for (int si = 0; si < GK; ++si) acc += wb[si] * (float)Cb[(int64_t)si * d + c];
        Cb[(int64_t)GK * d + c] = (bf16)acc;
    }
}

}  // namespace gqe
