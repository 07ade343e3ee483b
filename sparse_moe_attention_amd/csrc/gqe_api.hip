// libgqe: host side of the C ABI declared in include/gqe.h.
//
// Every argument is checked before the first HIP call. The caller's
// workspace is split into fixed buffers; kernels are enqueued in order on the
// caller's stream; nothing is allocated and nothing waits on the device.
//
// GQE forward (one stream, in order):
//   proj      x -> K, V^T (every group), Q_sh, router logits (+br)   [MFMA]
//   route     logits -> idx, w, per-chunk expert histogram
//   scan      histogram -> segment offsets and per-chunk bases
//   scatter   idx -> perm (token), dst (dense Qr row), per expert segment
//   grouped_q x[perm] Wq_e^T -> Qr[dst]                            [MFMA]
//   attention Qr, Q_sh over K/V -> hard slots and shared slot of C [MFMA]
//   combine   sum_s w_s * hard slot s -> weighted slot of C
//   proj      C Wo^T -> out                                          [MFMA]
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/gqe.h"
#include "attention.hpp"
#include "attention_bwd.hpp"
#include "backward.hpp"
#include "decode.hpp"
#include "gemm_launch.hpp"
#include "route.hpp"

using namespace gqe;

namespace {

// Sequence padding of the K / V^T buffers: whole key tiles of the forward
// and whole key blocks of the dK/dV kernel (its waves read their keys' rows).
constexpr int kKVPad = std::max({AttnShort::BKV, AttnShortF32::BKV, AttnLong::BKV, kBwdBKMax, kBwdBKVMax});

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Dims {
    int64_t B, T, D, N, Tpad, nC;
    int G, M, k, d, E, GK, s0;
    int variant;       // gqe_variant
    int slots;         // d-wide slots of the merged output C (Wo's input)
    int esz;
    bool f32;
    bool weighted_slot() const { return variant == GQE_FULL || variant == GQE_NO_SHARED; }
    bool shared_head() const { return variant != GQE_NO_SHARED; }
};

// Shape checks shared by every GQE entry point (no HIP call).
gqe_status check_shape(const gqe_shape* s, Dims* o) {
    if (s == nullptr) return GQE_ERR_NULL;
    if (s->B < 1 || s->T < 1 || s->D < 1 || s->G < 1 || s->M < 1 || s->k < 1) return GQE_ERR_SHAPE;
    if (s->k > s->M) return GQE_ERR_SHAPE;
    if (s->shared_kv_group < 0 || s->shared_kv_group >= s->G) return GQE_ERR_SHAPE;
    if (s->dtype != GQE_BF16 && s->dtype != GQE_F32) return GQE_ERR_UNSUPPORTED;
    if (s->variant < GQE_FULL || s->variant > GQE_NO_SHARED) return GQE_ERR_UNSUPPORTED;
    if (s->d_h != 32 && s->d_h != 64) return GQE_ERR_UNSUPPORTED;
    if (s->D % 64 != 0 || s->D > (int64_t)1 << 20) return GQE_ERR_UNSUPPORTED;
    if (s->M > 64 || (int64_t)s->G * s->M > 256) return GQE_ERR_UNSUPPORTED;
    if (s->B > ((int64_t)1 << 31) || s->T > ((int64_t)1 << 31)) return GQE_ERR_SHAPE;
    const int64_t N = s->B * s->T;
    const int64_t GK = (int64_t)s->G * s->k;
    const int slots = (int)GK + (s->variant == GQE_FULL ? 2 : 1);
    if (N * slots >= ((int64_t)1 << 31)) return GQE_ERR_SHAPE;   // int32 rows of Qr / perm
    Dims d;
    d.B = s->B; d.T = s->T; d.D = s->D; d.N = N;
    d.Tpad = (int64_t)align_up((size_t)s->T, kKVPad);
    d.nC = (N + kChunk - 1) / kChunk;
    d.G = s->G; d.M = s->M; d.k = s->k; d.d = s->d_h;
    d.E = s->G * s->M; d.GK = (int)GK; d.s0 = s->shared_kv_group;
    d.variant = s->variant; d.slots = slots;
    d.f32 = s->dtype == GQE_F32;
    d.esz = d.f32 ? 4 : 2;
    *o = d;
    return GQE_OK;
}

struct GqeWs {
    size_t logits, idx, w, hist, cbase, offsets, perm, dst, K, Vt, Qsh, Qr, C, total;
};

GqeWs gqe_layout(const Dims& d) {
    GqeWs L;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
    L.logits = take((size_t)d.N * d.E * 4);
    L.idx = take((size_t)d.N * d.GK * 4);
    L.w = take((size_t)d.N * d.GK * 4);
    L.hist = take((size_t)d.nC * d.E * 4);
    L.cbase = take((size_t)(d.nC + 1) * d.E * 4);
    L.offsets = take((size_t)(d.E + 1) * 4);
    L.perm = take((size_t)d.N * d.GK * 4);
    L.dst = take((size_t)d.N * d.GK * 4);
    L.K = take((size_t)d.G * d.B * d.Tpad * d.d * d.esz);
    L.Vt = take((size_t)d.G * d.B * d.Tpad * d.d * d.esz);
    L.Qsh = take((size_t)d.N * d.d * d.esz);
    L.Qr = take((size_t)d.N * d.GK * d.d * d.esz);
    L.C = take((size_t)d.N * d.slots * d.d * d.esz);
    L.total = o;
    return L;
}

inline char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
// Compute units of the current device (cached per device; 256 if unknown).
int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}
template <typename T, class Cfg>
void launch_proj(ProjArgs& a, int total_cols, hipStream_t st) {
    a.n_tiles_n = (total_cols + Cfg::BN - 1) / Cfg::BN;
    const int64_t n_m = (a.M_rows + Cfg::BM - 1) / Cfg::BM;
    // A persistent grid of the resident workgroups (the register budget's
    // waves per SIMD), in whole XCD rounds.
    const int64_t tiles = n_m * a.n_tiles_n * (a.n_split > 1 ? a.n_split : 1);
    const int per_cu = std::max(1, Cfg::WPE * 4 / (Cfg::WM * Cfg::WN));
    const int64_t grid = std::min<int64_t>(tiles, per_cu * (int64_t)align_up((size_t)device_cus(), 8));
    if constexpr (sizeof(T) == 2) launch_proj_gemm_bf16(a, (unsigned)grid, st);
    else launch_proj_gemm_f32(a, (unsigned)grid, st);
}

struct SegList {
    ProjArgs a;
    int cols = 0;
    void add(const void* W, int n_cols, void* out, int mode, int64_t ld_out, const float* bias,
             float scale = 1.f) {
        // A transposed block never shares a column tile with a row-major one.
        if (a.n_segs > 0 && (a.seg[a.n_segs - 1].mode == OUT_HEADS_T) != (mode == OUT_HEADS_T))
            cols = (int)align_up((size_t)cols, kProjClassAlign);
        ProjSeg& s = a.seg[a.n_segs++];
        s.W = W;
        s.out = out;
        s.bias = bias;
        s.ld_out = ld_out;
        s.col_begin = cols;
        s.n_cols = n_cols;
        s.mode = mode;
        s.scale = scale;
        cols += (int)align_up((size_t)n_cols, 8);
    }
};

SegList proj_base(const Dims& d, const void* A, int64_t lda, int64_t rows, int K) {
    SegList sl;
    std::memset(&sl.a, 0, sizeof(sl.a));
    sl.a.A = A;
    sl.a.lda = lda;
    sl.a.M_rows = rows;
    sl.a.T = d.T;
    sl.a.Tpad = d.Tpad;
    sl.a.Bt = (int)d.B;
    sl.a.K = K;
    sl.a.d = d.d;
    return sl;
}

void run_proj(const Dims& d, SegList& sl, hipStream_t st) {
    if (d.f32) launch_proj<float, ProjF32>(sl.a, sl.cols, st);
    else launch_proj<bf16, ProjBf16>(sl.a, sl.cols, st);
}

// A projection of at most kSkinnyMaxRows token rows (a decode step) in bf16:
// skinny_proj_kernel, one pass over the weights; larger ones take the tiled
// GEMM. Row-major outputs only, K a multiple of 32 (the callers' D and slot
// widths are).
constexpr int64_t kSkinnyMaxRows = 64;
void run_proj_rows(const Dims& d, SegList& sl, hipStream_t st) {
    if (d.f32 || sl.a.M_rows > kSkinnyMaxRows || sl.a.K % 32 != 0) {
        run_proj(d, sl, st);
        return;
    }
    sl.a.n_tiles_n = (sl.cols + 15) / 16;
    const int64_t n_m = (sl.a.M_rows + kSkinnyRows - 1) / kSkinnyRows;
    launch_skinny_proj(sl.a, (unsigned)(n_m * sl.a.n_tiles_n), st);
}

// Routing from the logits (route_kernel<0>): group widths 1, 2, 4, 8 and 16
// have their logits loaded into registers at once, others read them one by one.
void run_route(const Dims& d, const float* lg, int32_t* idx, float* w, int32_t* hist, hipStream_t st) {
    const int renorm = d.variant != GQE_WEIGHTED_CONCAT;
    const dim3 grid((unsigned)d.nC), blk(kRouteThreads);
    switch (d.M) {
        case 1: hipLaunchKernelGGL((route_kernel<0, 1>), grid, blk, 0, st, lg, idx, w, hist, d.N, d.G, d.M, d.k, renorm); break;
        case 2: hipLaunchKernelGGL((route_kernel<0, 2>), grid, blk, 0, st, lg, idx, w, hist, d.N, d.G, d.M, d.k, renorm); break;
        case 4: hipLaunchKernelGGL((route_kernel<0, 4>), grid, blk, 0, st, lg, idx, w, hist, d.N, d.G, d.M, d.k, renorm); break;
        case 8: hipLaunchKernelGGL((route_kernel<0, 8>), grid, blk, 0, st, lg, idx, w, hist, d.N, d.G, d.M, d.k, renorm); break;
        case 16: hipLaunchKernelGGL((route_kernel<0, 16>), grid, blk, 0, st, lg, idx, w, hist, d.N, d.G, d.M, d.k, renorm); break;
        default: hipLaunchKernelGGL((route_kernel<0, 0>), grid, blk, 0, st, lg, idx, w, hist, d.N, d.G, d.M, d.k, renorm);
    }
}

// Queries are stored pre-multiplied by log2(e)/sqrt(d): the attention kernel
// then works in log2 units with no per-score scaling.
float q_scale(const Dims& d) { return (float)(1.4426950408889634 / std::sqrt((double)d.d)); }

void run_grouped_q(const Dims& d, const void* x, const void* Wq, void* Qr, const int32_t* perm,
                   const int32_t* dst, const int32_t* cbase, hipStream_t st) {
    GroupArgs g;
    g.X = x; g.Wq = Wq; g.Qr = Qr; g.perm = perm; g.dst = dst; g.cbase = cbase;
    g.ldx = d.D; g.K = (int)d.D; g.d = d.d; g.E = d.E; g.nC = (int)d.nC;
    g.scale = q_scale(d);
    const int bm = d.f32 ? GrpF32::BM : GrpBf16::BM;
    g.n_t = (int)((d.N + bm - 1) / bm);
    // 8 * E * ceil(n_t / 8) workgroups: tile t = 8*(j/E) + hw%8 of expert j%E, j = hw/8.
    const dim3 grid((unsigned)(8 * (int64_t)d.E * ((g.n_t + 7) / 8)));
    if (d.f32) launch_grouped_q_f32(g, grid.x, st);
    else launch_grouped_q_bf16(g, grid.x, st);
}

// Attention tile shape by sequence length: AttnShort up to T = 256K, AttnLong
// beyond (measured on the 8-group d = 64 layer: AttnShort 1-3% ahead from
// T = 64K to 256K, even at 512K, AttnLong 34% ahead at 1M). fp32 layers (the
// small reference configuration) always take the short tile (AttnShortF32).
#ifndef GQE_ATTN_LONG_T
#define GQE_ATTN_LONG_T 262144
#endif
constexpr int64_t kAttnLongT = GQE_ATTN_LONG_T;
template <typename T, class Shape>
void launch_attention(const Dims& d, AttnArgs& a, hipStream_t st) {
    const bool xcls = a.Q1 != nullptr;
    a.n_o = (int)((d.T * a.R + Shape::BQ - 1) / Shape::BQ);
    a.n_x = xcls ? (int)((d.T * (a.R + 1) + Shape::BQ - 1) / Shape::BQ) : 0;
    const int64_t n_wg = d.B * ((int64_t)(xcls ? d.G - 1 : d.G) * a.n_o + a.n_x);
    const dim3 grid((unsigned)n_wg), block(Shape::NW * 64);
    if (d.d == 64) hipLaunchKernelGGL((attn_fwd_kernel<T, 64, Shape>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<T, 32, Shape>), grid, block, 0, st, a);
}

void run_attention(const Dims& d, AttnArgs& a, hipStream_t st) {
    a.T = d.T;
    a.Tpad = d.Tpad;
    a.Bt = (int)d.B;
    a.G = d.G;
    if (d.f32) launch_attention<float, AttnShortF32>(d, a, st);
    else if (d.T > kAttnLongT) launch_attention<bf16, AttnLong>(d, a, st);
    else launch_attention<bf16, AttnShort>(d, a, st);
}

// The merge step of the variant: the renormalised weighted slot (full,
// no-shared), the hard slots scaled in place by their weights (weighted
// concatenation), or nothing (hard concatenation).
void run_combine(const Dims& d, void* C, const float* w, hipStream_t st) {
    if (d.variant == GQE_HARD_CONCAT) return;
    const int64_t ldc = (int64_t)d.slots * d.d;
    const int scale_in_place = d.variant == GQE_WEIGHTED_CONCAT;
    const int64_t items = d.N * (d.d / 8);
    const dim3 grid((unsigned)((items + 255) / 256));
    if (d.f32)
        hipLaunchKernelGGL((combine_kernel<float>), grid, dim3(256), 0, st, (float*)C, w, d.N, ldc, d.GK, d.d,
                           scale_in_place);
    else
        hipLaunchKernelGGL((combine_kernel<bf16>), grid, dim3(256), 0, st, (bf16*)C, w, d.N, ldc, d.GK, d.d,
                           scale_in_place);
}

gqe_status last_hip() { return hipGetLastError() == hipSuccess ? GQE_OK : GQE_ERR_HIP; }

// Records events[i] (if any) on the stream: the instrumented entry points
// bracket every stage with these.
struct Marks {
    void* const* ev;
    hipStream_t st;
    void at(int i) const {
        if (ev != nullptr && ev[i] != nullptr) (void)hipEventRecord((hipEvent_t)ev[i], st);
    }
};

// Post-router part shared by gqe_attn_fwd and gqe_attn_fwd_routed:
// K/V/Q_sh projection, permutation, sparse Q, attention, combine, Wo.
gqe_status run_post_router(const Dims& d, const GqeWs& L, void* ws, const void* x, const void* Wq,
                           const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo,
                           const int32_t* idx, const float* w, void* out, void* C, hipStream_t st,
                           bool project_kv, const Marks& mk, float* lse = nullptr, int64_t lse_Lr = 0,
                           int64_t lse_Lx = 0) {
    if (project_kv) {
        SegList sl = proj_base(d, x, d.D, d.N, (int)d.D);
        sl.add(Wk, d.G * d.d, at(ws, L.K), OUT_HEADS, 0, nullptr);
        if (d.shared_head()) sl.add(Wq_sh, d.d, at(ws, L.Qsh), OUT_ROWS, d.d, nullptr, q_scale(d));
        sl.add(Wv, d.G * d.d, at(ws, L.Vt), OUT_HEADS_T, 0, nullptr);
        run_proj(d, sl, st);
    }
    int32_t* cbase = (int32_t*)at(ws, L.cbase);
    mk.at(2);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, (const int32_t*)at(ws, L.hist), cbase,
                       (int32_t*)at(ws, L.offsets), (int32_t*)nullptr, (int)d.nC, d.E);
    mk.at(3);
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)d.nC), dim3(kRouteThreads), 0, st, idx, (const int32_t*)cbase,
                       (int32_t*)at(ws, L.perm), (int32_t*)at(ws, L.dst), d.N, d.G, d.M, d.k);
    mk.at(4);
    run_grouped_q(d, x, Wq, at(ws, L.Qr), (const int32_t*)at(ws, L.perm), (const int32_t*)at(ws, L.dst),
                  cbase, st);
    AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.Q0 = at(ws, L.Qr);
    a.q0_ld = (int64_t)d.GK * d.d;
    a.Q1 = d.shared_head() ? at(ws, L.Qsh) : nullptr;
    a.q1_ld = d.d;
    a.K = at(ws, L.K);
    a.Vt = at(ws, L.Vt);
    a.O = C;
    a.o_ld = (int64_t)d.slots * d.d;
    a.R = d.k;                 // routed head j = g*k + r: hard slot j of C
    a.kv1 = d.s0;
    a.o1_col = (d.GK + (d.weighted_slot() ? 1 : 0)) * d.d;   // the shared slot is the last one
    a.lse = lse;
    a.lse_Lr = lse_Lr;
    a.lse_Lx = lse_Lx;
    mk.at(5);
    run_attention(d, a, st);
    mk.at(6);
    run_combine(d, C, w, st);
    mk.at(7);
    SegList so = proj_base(d, C, (int64_t)d.slots * d.d, d.N, d.slots * d.d);
    so.add(Wo, (int)d.D, out, OUT_ROWS, d.D, nullptr);
    run_proj(d, so, st);
    mk.at(8);
    return last_hip();
}

// ---------------------------------------------------------------------------
// Training: the forward that keeps what the backward needs, and the backward.
// ---------------------------------------------------------------------------
// The backward covers the full layer in bf16 (the other merge variants and
// fp32 layers are forward-only).
gqe_status check_train(const Dims& d) {
    if (d.f32 || d.variant != GQE_FULL) return GQE_ERR_UNSUPPORTED;
    return GQE_OK;
}

// The backward's gradient matrix dY [N, ccat_pad] (and its transpose): the
// gradients of everything x is projected to, side by side, so that
// dx = dY W_cat and dW_cat = dY^T x are one GEMM each:
//   [dQ of every expert (zero where not picked) | dK | dV | dQ_shared | dlogits | 0].
struct TrainWs {
    RowSpace rs;
    int64_t rows, Npad, ccat, ccat_pad, col_k, col_v, col_qsh, col_lg;
    int n_cs, ns_wo, ks_wo, ns_w, ks_w;
    int n_gs, n_gct;          // grouped dWq: splits per expert segment, column tiles
    // Forward state (lse) and backward buffers, after the forward's own layout.
    size_t lse, dlt, Qc, dOc, dw, dz, p, cs, dC, WoT, WcT, xT, doT, CT, V, dY, dYt, part, gpart, total;
};

constexpr int kRowPad = kBwdDqBQMax > 256 ? kBwdDqBQMax : 256;   // row-space runs pad to whole dQ row tiles
constexpr int kColsumRows = 256;

// Splits of a weight-gradient GEMM over its token contraction: about 1024
// workgroups (two rounds of MI355X's 256 CUs at two per CU), runs of at
// least 512 tokens. A function of the shape alone, so the workspace size and
// the summation order do not depend on the device.
void pick_splits(int64_t tiles, int64_t Kfull, int* ns, int* ks) {
    const int64_t want = (1024 + tiles - 1) / tiles;
    const int64_t cap = std::max<int64_t>(1, Kfull / 512);
    int64_t n = std::min(std::max<int64_t>(want, 1), cap);
    int64_t k = (int64_t)align_up((size_t)((Kfull + n - 1) / n), 64);
    n = (Kfull + k - 1) / k;
    *ns = (int)n;
    *ks = (int)k;
}

TrainWs train_layout(const Dims& d) {
    TrainWs L;
    L.rs.T = d.T;
    L.rs.Bt = (int32_t)d.B;
    L.rs.R = d.k;
    L.rs.s0 = d.s0;
    L.rs.Lr = (int64_t)align_up((size_t)(d.T * d.k), kRowPad);
    L.rs.Lx = (int64_t)align_up((size_t)(d.T * (d.k + 1)), kRowPad);
    L.rows = d.B * ((int64_t)d.G * L.rs.Lr + (L.rs.Lx - L.rs.Lr));
    L.Npad = (int64_t)align_up((size_t)d.N, 64);
    L.col_k = (int64_t)d.E * d.d;
    L.col_v = L.col_k + (int64_t)d.G * d.d;
    L.col_qsh = L.col_v + (int64_t)d.G * d.d;
    L.col_lg = L.col_qsh + d.d;
    L.ccat = L.col_lg + d.E;
    L.ccat_pad = (int64_t)align_up((size_t)L.ccat, 64);
    L.n_cs = (int)((d.N + kColsumRows - 1) / kColsumRows);
    const int64_t SD = (int64_t)d.slots * d.d;
    const int64_t t_wo = ((d.D + 127) / 128) * ((SD + 127) / 128);
    // The dense weight-gradient GEMM covers dY's columns from dK on; the
    // routed queries' dWq is the grouped kernel's.
    const int64_t wrows = L.ccat - L.col_k;
    const int64_t t_w = ((wrows + 127) / 128) * ((d.D + 127) / 128);
    pick_splits(t_wo, L.Npad, &L.ns_wo, &L.ks_wo);
    pick_splits(t_w, L.Npad, &L.ns_w, &L.ks_w);
    // Grouped dWq: about 1024 workgroups, segments split into runs of at
    // least 256 picks on average.
    L.n_gct = (int)((d.D + kDwBN - 1) / kDwBN);
    {
        const int64_t base = (int64_t)d.E * L.n_gct;
        const int64_t avg = d.N * d.GK / d.E;
        L.n_gs = (int)std::max<int64_t>(1, std::min<int64_t>((1024 + base - 1) / base, avg / 256));
    }

    size_t o = gqe_layout(d).total;
    auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
    const size_t rows = (size_t)L.rows;
    L.lse = take(rows * 4);
    L.dlt = take(rows * 4);
    L.Qc = take(rows * d.d * 2);
    L.dOc = take(rows * d.d * 2);
    L.dw = take((size_t)d.N * d.GK * 4);
    L.dz = take((size_t)d.N * d.E * 4);
    L.p = take((size_t)d.N * d.E * 4);
    L.cs = take((size_t)2 * L.n_cs * d.E * 4);
    L.dC = take((size_t)d.N * SD * 2);
    L.WoT = take((size_t)SD * d.D * 2);
    L.WcT = take((size_t)d.D * L.ccat_pad * 2);
    L.xT = take((size_t)d.D * L.Npad * 2);
    L.doT = take((size_t)d.D * L.Npad * 2);
    L.CT = take((size_t)SD * L.Npad * 2);
    L.V = take((size_t)d.G * d.B * d.Tpad * d.d * 2);
    L.dY = take((size_t)d.N * L.ccat_pad * 2);
    L.dYt = take((size_t)wrows * L.Npad * 2);
    L.part = take(std::max((size_t)L.ns_wo * d.D * SD, (size_t)L.ns_w * wrows * d.D) * 4);
    L.gpart = take((size_t)L.n_gs * d.E * d.d * d.D * 4);
    L.total = o;
    return L;
}

// dst[x][y] = src[y][x] (y < R, x < C), zero elsewhere in [Co x Ro]; z batches.
void run_transpose(const bf16* src, int64_t lds, int64_t R, int64_t C, bf16* dst, int64_t ldd, int64_t Ro,
                   int64_t Co, int z, int64_t zs, int64_t zd, hipStream_t st) {
    if (Ro <= 0 || Co <= 0) return;
    TrArgs t;
    t.src = src; t.dst = dst; t.lds = lds; t.ldd = ldd;
    t.R = R; t.C = C; t.Ro = Ro; t.Co = Co; t.zs = zs; t.zd = zd;
    const dim3 grid((unsigned)(((Ro + 63) / 64) * ((Co + 63) / 64)), (unsigned)z);
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, t);
}

// Projection-engine GEMM out = A W^T over plain matrices (no head layouts).
SegList gemm_base(const void* A, int64_t lda, int64_t rows, int K) {
    SegList sl;
    std::memset(&sl.a, 0, sizeof(sl.a));
    sl.a.A = A;
    sl.a.lda = lda;
    sl.a.M_rows = rows;
    sl.a.T = rows;
    sl.a.Tpad = rows;
    sl.a.Bt = 1;
    sl.a.K = K;
    sl.a.d = 64;
    return sl;
}

// Weight gradient through split-K: part[s] = A_s W_s^T, then a fixed-order
// sum scattered to the destinations (row ranges of the product).
void run_wgrad(const void* A, int64_t lda, int64_t rows, const void* W, int64_t cols, int64_t K, int ns, int ks,
               float* part, const RedDst* dst, int n_dst, hipStream_t st) {
    SegList sl = gemm_base(A, lda, rows, (int)K);
    sl.add(W, (int)cols, part, OUT_ROWS_F32, cols, nullptr);
    sl.a.n_split = ns;
    sl.a.k_split = ks;
    sl.a.split_stride = rows * cols;
    launch_proj<bf16, ProjBf16>(sl.a, sl.cols, st);
    RedArgs r;
    std::memset(&r, 0, sizeof(r));
    r.part = part;
    r.split_stride = rows * cols;
    r.rows = rows;
    r.cols = cols;
    r.n_split = ns;
    r.n_dst = n_dst;
    for (int i = 0; i < n_dst; ++i) r.dst[i] = dst[i];
    const int64_t items = rows * (cols / 4);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st, r);
}

// Zero K rows and V^T columns of tokens in [T, Tpad): K (whose columns the dQ
// kernel contracts over keys) and the row-major V copy then hold zeros there.
__global__ void kv_pad_kernel(bf16* K, bf16* Vt, int64_t T, int64_t Tpad, int Bt, int d) {
    const int g = blockIdx.x / Bt, b = blockIdx.x % Bt;
    const int64_t n_pad = Tpad - T;
    bf16* kp = K + (((int64_t)g * Bt + b) * Tpad + T) * d;
    for (int64_t i = threadIdx.x; i < n_pad * d; i += blockDim.x) kp[i] = (bf16)0.f;
    const int64_t vrow = (int64_t)Bt * Tpad;
    for (int64_t i = threadIdx.x; i < n_pad * d; i += blockDim.x) {
        const int64_t c = i / n_pad, t = T + i % n_pad;
        Vt[((int64_t)g * d + c) * vrow + (int64_t)b * Tpad + t] = (bf16)0.f;
    }
}

gqe_status bwd_impl(const gqe_shape* s, const void* x, const void* Wr, const void* Wq, const void* Wk,
                    const void* Wv, const void* Wq_sh, const void* Wo, const void* dout, float aux_coef, float* dx,
                    float* dWr, float* dbr, float* dWq, float* dWk, float* dWv, float* dWq_sh, float* dWo,
                    float* aux_loss, void* ws, size_t ws_bytes, void* stream, void* const* events) {
    Dims d;
    gqe_status rc = check_shape(s, &d);
    if (rc != GQE_OK) return rc;
    if ((rc = check_train(d)) != GQE_OK) return rc;
    if (!x || !Wr || !Wq || !Wk || !Wv || !Wq_sh || !Wo || !dout || !dx || !dWr || !dWq || !dWk || !dWv ||
        !dWq_sh || !dWo || !ws)
        return GQE_ERR_NULL;
    if (!aligned16(x) || !aligned16(Wr) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) ||
        !aligned16(Wq_sh) || !aligned16(Wo) || !aligned16(dout) || !aligned16(dx) || !aligned16(dWr) ||
        !aligned16(dWq) || !aligned16(dWk) || !aligned16(dWv) || !aligned16(dWq_sh) || !aligned16(dWo) ||
        !aligned16(ws) || (dbr && !aligned16(dbr)))
        return GQE_ERR_ALIGN;
    if (!std::isfinite(aux_coef)) return GQE_ERR_SHAPE;
    const GqeWs F = gqe_layout(d);
    const TrainWs L = train_layout(d);
    if (ws_bytes < L.total) return GQE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const Marks mk{events, st};
    const int64_t SD = (int64_t)d.slots * d.d, N = d.N, D = d.D, dh = d.d;
    const int64_t vrow = d.B * d.Tpad;
    auto B = [&](size_t off) { return (bf16*)at(ws, off); };
    auto F32 = [&](size_t off) { return (float*)at(ws, off); };

    mk.at(0);
    // Operand layouts: transposed weights and token-contiguous activations.
    run_transpose((const bf16*)Wo, SD, D, SD, B(L.WoT), D, D, SD, 1, 0, 0, st);
    bf16* wct = B(L.WcT);
    run_transpose((const bf16*)Wq, D, (int64_t)d.E * dh, D, wct, L.ccat_pad, (int64_t)d.E * dh, D, 1, 0, 0, st);
    run_transpose((const bf16*)Wk, D, (int64_t)d.G * dh, D, wct + L.col_k, L.ccat_pad, (int64_t)d.G * dh, D, 1, 0, 0, st);
    run_transpose((const bf16*)Wv, D, (int64_t)d.G * dh, D, wct + L.col_v, L.ccat_pad, (int64_t)d.G * dh, D, 1, 0, 0, st);
    run_transpose((const bf16*)Wq_sh, D, dh, D, wct + L.col_qsh, L.ccat_pad, dh, D, 1, 0, 0, st);
    run_transpose((const bf16*)Wr, D, d.E, D, wct + L.col_lg, L.ccat_pad, L.ccat_pad - L.col_lg, D, 1, 0, 0, st);
    run_transpose((const bf16*)x, D, N, D, B(L.xT), L.Npad, L.Npad, D, 1, 0, 0, st);
    run_transpose((const bf16*)dout, D, N, D, B(L.doT), L.Npad, L.Npad, D, 1, 0, 0, st);
    run_transpose(B(F.C), SD, N, SD, B(L.CT), L.Npad, L.Npad, SD, 1, 0, 0, st);
    if (d.Tpad > d.T)
        hipLaunchKernelGGL(kv_pad_kernel, dim3((unsigned)(d.G * d.B)), dim3(256), 0, st, B(F.K), B(F.Vt), d.T, d.Tpad,
                           (int)d.B, d.d);
    run_transpose(B(F.Vt), vrow, dh, vrow, B(L.V), dh, dh, vrow, d.G, vrow * dh, vrow * dh, st);
    mk.at(1);

    // Slot gradients dC = dout Wo, and dWo = dout^T C.
    {
        SegList sl = gemm_base(dout, D, N, (int)D);
        sl.add(B(L.WoT), (int)SD, B(L.dC), OUT_ROWS, SD, nullptr);
        launch_proj<bf16, ProjBf16>(sl.a, sl.cols, st);
        const RedDst dst{dWo, 0, D};
        run_wgrad(B(L.doT), L.Npad, D, B(L.CT), SD, L.Npad, L.ns_wo, L.ks_wo, F32(L.part), &dst, 1, st);
    }
    mk.at(2);

    // Attention rows: dO, dw, delta and the compact copies.
    {
        PrepArgs pa;
        pa.Qr = B(F.Qr); pa.Qsh = B(F.Qsh); pa.C = B(F.C); pa.dC = B(L.dC);
        pa.w = F32(F.w);
        pa.Qc = B(L.Qc); pa.dOc = B(L.dOc);
        pa.lse = F32(L.lse); pa.dlt = F32(L.dlt); pa.dw = F32(L.dw);
        pa.rs = L.rs;
        pa.ldc = SD;
        pa.G = d.G; pa.k = d.k; pa.d = d.d;
        pa.wcol = d.GK * d.d;
        pa.shcol = (d.GK + 1) * d.d;
        const dim3 grid((unsigned)(L.rs.Lx / 64), (unsigned)(d.G * d.B));
        if (d.d == 64) hipLaunchKernelGGL(prep_kernel<64>, grid, dim3(256), 0, st, pa);
        else hipLaunchKernelGGL(prep_kernel<32>, grid, dim3(256), 0, st, pa);
    }
    // Router: dlogits (and the zero columns of unpicked experts), dbr, balancing loss.
    {
        RouterBwdArgs ra;
        ra.logits = F32(F.logits);
        ra.idx = (const int32_t*)at(ws, F.idx);
        ra.w = F32(F.w);
        ra.dw = F32(L.dw);
        ra.offsets = (const int32_t*)at(ws, F.offsets);
        ra.dz = F32(L.dz);
        ra.p = F32(L.p);
        ra.dY = B(L.dY);
        ra.N = N;
        ra.ldy = L.ccat_pad;
        ra.G = d.G; ra.M = d.M; ra.k = d.k; ra.d = d.d;
        ra.lg_col = (int)L.col_lg;
        ra.pad_col = (int)L.ccat;
        ra.coef = aux_coef;
        // dQ columns of every expert start at zero; the dQ kernel writes the picked ones.
        const int64_t zq = N * ((int64_t)d.E * d.d / 8);
        hipLaunchKernelGGL(zero_cols_kernel, dim3((unsigned)((zq + 255) / 256)), dim3(256), 0, st, B(L.dY), N,
                           (int64_t)d.E * d.d, L.ccat_pad);
        hipLaunchKernelGGL(router_bwd_kernel, dim3((unsigned)((N + 63) / 64)), dim3(64), 0, st, ra);
        hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)L.n_cs), dim3(256), 0, st, (const float*)F32(L.dz),
                           (const float*)F32(L.p), F32(L.cs), N, d.E, kColsumRows);
        hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(256), 0, st, (const float*)F32(L.cs), L.n_cs,
                           (const int32_t*)at(ws, F.offsets), N, d.G, d.M, d.k, aux_coef, dbr, aux_loss);
    }
    mk.at(3);

    // Attention backward.
    AttnBwdArgs ab;
    ab.Q = B(L.Qc); ab.dO = B(L.dOc);
    ab.lse = F32(L.lse); ab.dlt = F32(L.dlt);
    ab.K = B(F.K); ab.V = B(L.V);
    ab.dY = B(L.dY);
    ab.idx = (const int32_t*)at(ws, F.idx);
    ab.ldy = L.ccat_pad;
    ab.Tpad = d.Tpad;
    ab.rs = L.rs;
    ab.G = d.G; ab.M = d.M; ab.k = d.k;
    ab.colK = (int)L.col_k; ab.colV = (int)L.col_v; ab.colQsh = (int)L.col_qsh;
    {
        const int bk = d.d == 64 ? bwd_bk<64>() : bwd_bk<32>();
        ab.n_tiles = (int)((d.T + bk - 1) / bk);
        const dim3 grid((unsigned)bwd_jobs(L.rs, (int)d.G, ab.n_tiles, ab.n_tiles));
        if (d.d == 64) hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, grid, dim3(bwd_nw<64>() * 64), 0, st, ab);
        else hipLaunchKernelGGL(attn_bwd_dkdv_kernel<32>, grid, dim3(bwd_nw<32>() * 64), 0, st, ab);
    }
    mk.at(4);
    {
        // Long sequences (d = 64) take the 256-row shape, as the forward does.
        const bool lng = d.d == 64 && d.T > kAttnLongT;
        const int bq = lng ? DqLong::BQ : DqShort::BQ;
        ab.n_tiles = (int)((d.T * (d.k + 1) + bq - 1) / bq);
        const dim3 grid((unsigned)bwd_jobs(L.rs, (int)d.G, (d.T * d.k + bq - 1) / bq, ab.n_tiles));
        if (lng) hipLaunchKernelGGL((attn_bwd_dq_kernel<64, DqLong>), grid, dim3(DqLong::NW * 64), 0, st, ab);
        else if (d.d == 64) hipLaunchKernelGGL((attn_bwd_dq_kernel<64, DqShort>), grid, dim3(DqShort::NW * 64), 0, st, ab);
        else hipLaunchKernelGGL((attn_bwd_dq_kernel<32, DqShort>), grid, dim3(DqShort::NW * 64), 0, st, ab);
    }
    mk.at(5);

    // dx = dY W_cat, dW_cat = dY^T x (dWq grouped by expert, the rest dense).
    const int64_t wrows = L.ccat - L.col_k;
    run_transpose(B(L.dY) + L.col_k, L.ccat_pad, N, wrows, B(L.dYt), L.Npad, L.Npad, wrows, 1, 0, 0, st);
    {
        SegList sl = gemm_base(B(L.dY), L.ccat_pad, N, (int)L.ccat_pad);
        sl.add(B(L.WcT), (int)D, dx, OUT_ROWS_F32, D, nullptr);
        launch_proj<bf16, ProjBf16>(sl.a, sl.cols, st);
    }
    mk.at(6);
    {
        GroupDwArgs ga;
        ga.dY = B(L.dY);
        ga.X = (const bf16*)x;
        ga.perm = (const int32_t*)at(ws, F.perm);
        ga.cbase = (const int32_t*)at(ws, F.cbase);
        ga.part = F32(L.gpart);
        ga.ldy = L.ccat_pad;
        ga.split_stride = (int64_t)d.E * dh * D;
        ga.D = (int32_t)D; ga.E = d.E; ga.nC = (int32_t)d.nC; ga.S = L.n_gs; ga.n_ct = L.n_gct;
        const dim3 grid((unsigned)((int64_t)L.n_gs * d.E * L.n_gct));
        if (dh == 64) hipLaunchKernelGGL(grouped_dw_kernel<64>, grid, dim3(256), 0, st, ga);
        else hipLaunchKernelGGL(grouped_dw_kernel<32>, grid, dim3(256), 0, st, ga);
        RedArgs r;
        std::memset(&r, 0, sizeof(r));
        r.part = F32(L.gpart);
        r.split_stride = ga.split_stride;
        r.rows = (int64_t)d.E * dh;
        r.cols = D;
        r.n_split = L.n_gs;
        r.n_dst = 1;
        r.dst[0] = RedDst{dWq, 0, (int64_t)d.E * dh};
        const int64_t items = r.rows * (D / 4);
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st, r);
        const RedDst dst[4] = {{dWk, 0, (int64_t)d.G * dh},
                               {dWv, L.col_v - L.col_k, (int64_t)d.G * dh},
                               {dWq_sh, L.col_qsh - L.col_k, dh},
                               {dWr, L.col_lg - L.col_k, d.E}};
        run_wgrad(B(L.dYt), L.Npad, wrows, B(L.xT), D, L.Npad, L.ns_w, L.ks_w, F32(L.part), dst, 4, st);
    }
    mk.at(7);
    return last_hip();
}

// idx_in (training only, may be null): the caller's picks replace the router's.
gqe_status fwd_impl(const gqe_shape* s, const void* x, const void* Wr, const float* br, const void* Wq,
                    const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo, void* out, int32_t* idx_out,
                    float* w_out, void* ws, size_t ws_bytes, void* stream, void* const* events, bool train,
                    const int32_t* idx_in = nullptr) {
    Dims d;
    gqe_status rc = check_shape(s, &d);
    if (rc != GQE_OK) return rc;
    if (!x || !Wr || !Wq || !Wk || !Wv || !Wq_sh || !Wo || !out || !ws) return GQE_ERR_NULL;
    if (!aligned16(x) || !aligned16(Wr) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) ||
        !aligned16(Wq_sh) || !aligned16(Wo) || !aligned16(out) || !aligned16(ws) || (br && !aligned16(br)) ||
        (idx_out && !aligned16(idx_out)) || (w_out && !aligned16(w_out)) || (idx_in && !aligned16(idx_in)))
        return GQE_ERR_ALIGN;
    if (train && (rc = check_train(d)) != GQE_OK) return rc;
    const GqeWs L = gqe_layout(d);
    const TrainWs TL = train_layout(d);
    if (ws_bytes < (train ? TL.total : L.total)) return GQE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    // Training keeps the routing in ws for the backward (copied out below).
    int32_t* idx = (idx_out && !train) ? idx_out : (int32_t*)at(ws, L.idx);
    float* w = (w_out && !train) ? w_out : (float*)at(ws, L.w);
    float* lg = (float*)at(ws, L.logits);
    const Marks mk{events, st};
    mk.at(0);
    // One pass over x: K, V^T, Q_sh and the router logits.
    SegList sl = proj_base(d, x, d.D, d.N, (int)d.D);
    sl.add(Wk, d.G * d.d, at(ws, L.K), OUT_HEADS, 0, nullptr);
    if (d.shared_head()) sl.add(Wq_sh, d.d, at(ws, L.Qsh), OUT_ROWS, d.d, nullptr, q_scale(d));
    sl.add(Wr, d.E, lg, OUT_ROWS_F32, d.E, br);
    sl.add(Wv, d.G * d.d, at(ws, L.Vt), OUT_HEADS_T, 0, nullptr);
    run_proj(d, sl, st);
    mk.at(1);
    if (idx_in != nullptr) {
        hipLaunchKernelGGL(inject_route_kernel, dim3((unsigned)((d.N + 255) / 256)), dim3(256), 0, st,
                           (const float*)lg, idx_in, idx, w, d.N, d.G, d.M, d.k);
        hipLaunchKernelGGL((route_kernel<1, 0>), dim3((unsigned)d.nC), dim3(kRouteThreads), 0, st,
                           (const float*)nullptr, idx, (float*)nullptr, (int32_t*)at(ws, L.hist), d.N, d.G, d.M, d.k,
                           1);
    } else {
        run_route(d, lg, idx, w, (int32_t*)at(ws, L.hist), st);
    }
    rc = run_post_router(d, L, ws, x, Wq, Wk, Wv, Wq_sh, Wo, idx, w, out, at(ws, L.C), st, false, mk,
                         train ? (float*)at(ws, TL.lse) : nullptr, TL.rs.Lr, TL.rs.Lx);
    if (rc != GQE_OK || !train) return rc;
    const size_t picks = (size_t)d.N * d.GK;
    if (idx_out && hipMemcpyAsync(idx_out, idx, picks * 4, hipMemcpyDeviceToDevice, st) != hipSuccess) return GQE_ERR_HIP;
    if (w_out && hipMemcpyAsync(w_out, w, picks * 4, hipMemcpyDeviceToDevice, st) != hipSuccess) return GQE_ERR_HIP;
    return GQE_OK;
}

// ---------------------------------------------------------------------------
// Decode: one new token per sequence over a dense KV cache.
// ---------------------------------------------------------------------------
// The per-token part (projections, routing, permutation, sparse Q) runs as the
// layer does on B tokens of length-1 sequences; the cache part has capacity T.
gqe_status check_decode(const gqe_shape* s, Dims* cache, Dims* tok) {
    gqe_status rc = check_shape(s, cache);
    if (rc != GQE_OK) return rc;
    if (cache->f32 || cache->variant != GQE_FULL) return GQE_ERR_UNSUPPORTED;
    if (s->T % 32 != 0) return GQE_ERR_SHAPE;                // 8-key V^T pieces never straddle T
    // The attention reads one group's V^T (d x B*T) through a 32-bit buffer view.
    if ((int64_t)s->d_h * s->B * s->T * 2 > (int64_t)UINT32_MAX) return GQE_ERR_SHAPE;
    gqe_shape t = *s;
    t.T = 1;
    return check_shape(&t, tok);
}

struct DecodeWs {
    GqeWs tok;
    size_t Kn, Vn, part_o, part_ml, total;
    int cw, n_ch, R16;    // keys per wave of the cache attention, chunks per sequence, head slots
};

DecodeWs decode_layout(const Dims& c, const Dims& t) {
    DecodeWs L;
    L.tok = gqe_layout(t);
    // The largest of 512, 256, 128 and 64 keys per wave that still launches
    // 1024 workgroups (four per CU): a short cache takes shorter chunks (at
    // 2K positions 64 keys per wave: 13.5 us against 15.1 with 128).
    L.cw = 512;
    while (L.cw > 64 && (int64_t)c.B * c.G * ((c.T + kDecNW * L.cw - 1) / (kDecNW * L.cw)) < 1024) L.cw /= 2;
    L.n_ch = (int)((c.T + kDecNW * L.cw - 1) / (kDecNW * L.cw));
    L.R16 = (int)align_up((size_t)(c.k + 1), 16);
    size_t o = L.tok.total;
    auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
    L.Kn = take((size_t)t.N * c.G * c.d * 2);
    L.Vn = take((size_t)t.N * c.G * c.d * 2);
    const size_t heads = (size_t)c.B * c.G * L.n_ch * L.R16;
    L.part_o = take(heads * c.d * 4);
    L.part_ml = take(heads * 2 * 4);
    L.total = o;
    return L;
}

gqe_status decode_impl(const gqe_shape* s, const int32_t* pos, const void* x, const void* Wr, const float* br,
                       const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo, void* k_cache,
                       void* vt_cache, void* out, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                       void* stream, void* const* events) {
    Dims c, t;
    gqe_status rc = check_decode(s, &c, &t);
    if (rc != GQE_OK) return rc;
    if (!pos || !x || !Wr || !Wq || !Wk || !Wv || !Wq_sh || !Wo || !k_cache || !vt_cache || !out || !ws)
        return GQE_ERR_NULL;
    if (!aligned16(pos) || !aligned16(x) || !aligned16(Wr) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) ||
        !aligned16(Wq_sh) || !aligned16(Wo) || !aligned16(k_cache) || !aligned16(vt_cache) || !aligned16(out) ||
        !aligned16(ws) || (br && !aligned16(br)) || (idx_out && !aligned16(idx_out)) || (w_out && !aligned16(w_out)))
        return GQE_ERR_ALIGN;
    const DecodeWs L = decode_layout(c, t);
    if (ws_bytes < L.total) return GQE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const Marks mk{events, st};
    const GqeWs& F = L.tok;
    int32_t* idx = idx_out ? idx_out : (int32_t*)at(ws, F.idx);
    float* w = w_out ? w_out : (float*)at(ws, F.w);
    float* lg = (float*)at(ws, F.logits);
    mk.at(0);
    // New token: K, V rows, the shared head's query, router logits.
    {
        SegList sl = proj_base(t, x, t.D, t.N, (int)t.D);
        sl.add(Wk, c.G * c.d, at(ws, L.Kn), OUT_ROWS, (int64_t)c.G * c.d, nullptr);
        sl.add(Wq_sh, c.d, at(ws, F.Qsh), OUT_ROWS, c.d, nullptr, q_scale(c));
        sl.add(Wr, c.E, lg, OUT_ROWS_F32, c.E, br);
        sl.add(Wv, c.G * c.d, at(ws, L.Vn), OUT_ROWS, (int64_t)c.G * c.d, nullptr);
        run_proj_rows(t, sl, st);
    }
    {
        DecTokArgs ta;
        ta.logits = lg;
        ta.x = (const bf16*)x;
        ta.Wq = (const bf16*)Wq;
        ta.Kn = (const bf16*)at(ws, L.Kn);
        ta.Vn = (const bf16*)at(ws, L.Vn);
        ta.pos = pos;
        ta.idx = idx;
        ta.w = w;
        ta.Qr = (bf16*)at(ws, F.Qr);
        ta.kc = (bf16*)k_cache;
        ta.vtc = (bf16*)vt_cache;
        ta.T = c.T;
        ta.D = c.D;
        ta.Bt = (int)c.B;
        ta.G = c.G;
        ta.M = c.M;
        ta.k = c.k;
        ta.d = c.d;
        ta.qscale = q_scale(c);
        const dim3 grid((unsigned)(c.B * c.G * c.k * (c.d / 16))), blk(256);
        switch (c.M) {
            case 1: hipLaunchKernelGGL(decode_token_kernel<1>, grid, blk, 0, st, ta); break;
            case 2: hipLaunchKernelGGL(decode_token_kernel<2>, grid, blk, 0, st, ta); break;
            case 4: hipLaunchKernelGGL(decode_token_kernel<4>, grid, blk, 0, st, ta); break;
            case 8: hipLaunchKernelGGL(decode_token_kernel<8>, grid, blk, 0, st, ta); break;
            case 16: hipLaunchKernelGGL(decode_token_kernel<16>, grid, blk, 0, st, ta); break;
            default: hipLaunchKernelGGL(decode_token_kernel<0>, grid, blk, 0, st, ta);
        }
    }
    mk.at(1);
    DecodeArgs a;
    a.Qr = (const bf16*)at(ws, F.Qr);
    a.Qsh = (const bf16*)at(ws, F.Qsh);
    a.K = (const bf16*)k_cache;
    a.Vt = (const bf16*)vt_cache;
    a.pos = pos;
    a.part_o = (float*)at(ws, L.part_o);
    a.part_ml = (float*)at(ws, L.part_ml);
    a.T = c.T;
    a.Bt = (int)c.B;
    a.G = c.G;
    a.k = c.k;
    a.s0 = c.s0;
    a.d = c.d;
    a.n_ch = L.n_ch;
    a.R16 = L.R16;
    const dim3 grid((unsigned)((int64_t)c.B * c.G * L.n_ch));
    const dim3 blk(kDecNW * 64);
    if (c.d == 64) {
        if (L.cw == 512) hipLaunchKernelGGL((attn_decode_kernel<64, 512>), grid, blk, 0, st, a);
        else if (L.cw == 256) hipLaunchKernelGGL((attn_decode_kernel<64, 256>), grid, blk, 0, st, a);
        else if (L.cw == 128) hipLaunchKernelGGL((attn_decode_kernel<64, 128>), grid, blk, 0, st, a);
        else hipLaunchKernelGGL((attn_decode_kernel<64, 64>), grid, blk, 0, st, a);
    } else {
        if (L.cw == 512) hipLaunchKernelGGL((attn_decode_kernel<32, 512>), grid, blk, 0, st, a);
        else if (L.cw == 256) hipLaunchKernelGGL((attn_decode_kernel<32, 256>), grid, blk, 0, st, a);
        else if (L.cw == 128) hipLaunchKernelGGL((attn_decode_kernel<32, 128>), grid, blk, 0, st, a);
        else hipLaunchKernelGGL((attn_decode_kernel<32, 64>), grid, blk, 0, st, a);
    }
    mk.at(2);
    bf16* C = (bf16*)at(ws, F.C);
    const int64_t ldc = (int64_t)c.slots * c.d;
    const int comb_waves = std::min(c.GK + 1, kDecCombMaxWaves);
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)c.B), dim3(comb_waves * 64), 0, st,
                       (const float*)a.part_o, (const float*)a.part_ml, (const float*)w, pos, C, c.G, c.k, c.s0, c.d,
                       L.n_ch, kDecNW * L.cw, L.R16, ldc, c.T);
    SegList so = proj_base(t, C, ldc, t.N, (int)ldc);
    so.add(Wo, (int)c.D, out, OUT_ROWS, c.D, nullptr);
    run_proj_rows(t, so, st);
    mk.at(3);
    return last_hip();
}

}  // namespace

// ---------------------------------------------------------------------------
// Allocation-free forward: the workspace lives in a static device array.
// ---------------------------------------------------------------------------
// Each device the library runs on holds its own copy of `scratch` from the
// code object's load until the process ends. Host code must never pass the
// array's name to a kernel or a copy (on the host it is only a stand-in for
// the symbol): scratch_base() looks up this device's address once and every
// launch takes that pointer.
static __device__ __align__(256) char scratch[GQE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_base[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
gqe_status scratch_base(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_base[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GQE_ERR_HIP;
        g_scratch_base[dev] = p;
    }
    *out = g_scratch_base[dev];
    return GQE_OK;
}

}  // namespace

// Sustained matrix-core rate: each wave keeps eight independent accumulator
// chains of v_mfma_f32_16x16x32_bf16 on fixed register operands (distinct,
// non-trivial bf16 values per lane), so the loop is matrix work only. Two
// or more waves per SIMD keep the accumulators in ordinary VGPRs (a
// one-wave budget would put them in AGPRs, which the compiler then shuffles).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 4))) void mfma_probe_kernel(int iters, float* out) {
    const int lane = threadIdx.x & 63;
    Frag<bf16> a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a.v[i] = (bf16)(0.25f + 0.01f * (float)((lane * 7 + i * 3) % 29));
        b.v[i] = (bf16)(0.5f - 0.013f * (float)((lane * 5 + i * 11) % 31));
    }
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, (float)j};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mma16(a, b, acc[j]);
    }
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) t += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    __shared__ float red[4];
    // lane 0 of each wave: its lane's share (enough to keep the work live)
    if (lane == 0) red[threadIdx.x >> 6] = t;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

extern "C" {

size_t gqe_workspace_bytes(const gqe_shape* s) {
    Dims d;
    if (check_shape(s, &d) != GQE_OK) return 0;
    return gqe_layout(d).total;
}

gqe_status gqe_route(const gqe_shape* s, const void* x, const void* Wr, const float* br, int32_t* idx,
                     float* w, float* logits, int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    gqe_status rc = check_shape(s, &d);
    if (rc != GQE_OK) return rc;
    if (!x || !Wr || !idx || !w || !ws) return GQE_ERR_NULL;
    if (!aligned16(x) || !aligned16(Wr) || !aligned16(idx) || !aligned16(w) || !aligned16(ws) ||
        (br && !aligned16(br)) || (logits && !aligned16(logits)) || (counts && !aligned16(counts)))
        return GQE_ERR_ALIGN;
    const GqeWs L = gqe_layout(d);
    if (ws_bytes < L.total) return GQE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    float* lg = logits ? logits : (float*)at(ws, L.logits);
    SegList sl = proj_base(d, x, d.D, d.N, (int)d.D);
    sl.add(Wr, d.E, lg, OUT_ROWS_F32, d.E, br);
    run_proj(d, sl, st);
    int32_t* hist = (int32_t*)at(ws, L.hist);
    run_route(d, lg, idx, w, hist, st);
    if (counts)
        hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, (const int32_t*)hist,
                           (int32_t*)at(ws, L.cbase), (int32_t*)at(ws, L.offsets), counts, (int)d.nC, d.E);
    return last_hip();
}

gqe_status gqe_attn_fwd_routed(const gqe_shape* s, const void* x, const void* Wq, const void* Wk,
                               const void* Wv, const void* Wq_sh, const void* Wo, const int32_t* idx,
                               const float* w, void* out, void* slots_out, void* ws, size_t ws_bytes,
                               void* stream) {
    Dims d;
    gqe_status rc = check_shape(s, &d);
    if (rc != GQE_OK) return rc;
    if (!x || !Wq || !Wk || !Wv || !Wq_sh || !Wo || !idx || !w || !out || !ws) return GQE_ERR_NULL;
    if (!aligned16(x) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) || !aligned16(Wq_sh) ||
        !aligned16(Wo) || !aligned16(idx) || !aligned16(w) || !aligned16(out) || !aligned16(ws) ||
        (slots_out && !aligned16(slots_out)))
        return GQE_ERR_ALIGN;
    const GqeWs L = gqe_layout(d);
    if (ws_bytes < L.total) return GQE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL((route_kernel<1, 0>), dim3((unsigned)d.nC), dim3(kRouteThreads), 0, st, (const float*)nullptr,
                       const_cast<int32_t*>(idx), (float*)nullptr, (int32_t*)at(ws, L.hist), d.N, d.G, d.M, d.k, 1);
    void* C = slots_out ? slots_out : at(ws, L.C);
    return run_post_router(d, L, ws, x, Wq, Wk, Wv, Wq_sh, Wo, idx, w, out, C, st, true, Marks{nullptr, st});
}

gqe_status gqe_attn_fwd_timed(const gqe_shape* s, const void* x, const void* Wr, const float* br,
                              const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo,
                              void* out, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes, void* stream,
                              void* const* events) {
    return fwd_impl(s, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, idx_out, w_out, ws, ws_bytes, stream, events, false);
}

gqe_status gqe_attn_fwd(const gqe_shape* s, const void* x, const void* Wr, const float* br, const void* Wq,
                        const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo, void* out,
                        int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes, void* stream) {
    return gqe_attn_fwd_timed(s, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, idx_out, w_out, ws, ws_bytes, stream,
                              nullptr);
}

gqe_status gqe_attn_fwd_noalloc(const gqe_shape* s, const void* x, const void* Wr, const float* br,
                                const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo,
                                void* out, int32_t* idx_out, float* w_out, void* stream) {
    // Every argument check of gqe_attn_fwd, and the scratch bound, before any HIP call.
    Dims d;
    gqe_status rc = check_shape(s, &d);
    if (rc != GQE_OK) return rc;
    if (!x || !Wr || !Wq || !Wk || !Wv || !Wq_sh || !Wo || !out) return GQE_ERR_NULL;
    if (!aligned16(x) || !aligned16(Wr) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) ||
        !aligned16(Wq_sh) || !aligned16(Wo) || !aligned16(out) || (br && !aligned16(br)) ||
        (idx_out && !aligned16(idx_out)) || (w_out && !aligned16(w_out)))
        return GQE_ERR_ALIGN;
    if (gqe_layout(d).total > (size_t)GQE_NOALLOC_SCRATCH_BYTES) return GQE_ERR_SCRATCH;
    void* ws = nullptr;
    if ((rc = scratch_base(&ws)) != GQE_OK) return rc;
    // The forward writes every workspace entry it reads (K/V rows past T are
    // masked, V^T columns past T zeroed in LDS), so the previous call's
    // contents need no clearing.
    return fwd_impl(s, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, idx_out, w_out, ws, (size_t)GQE_NOALLOC_SCRATCH_BYTES,
                    stream, nullptr, false);
}

size_t gqe_train_workspace_bytes(const gqe_shape* s) {
    Dims d;
    if (check_shape(s, &d) != GQE_OK || check_train(d) != GQE_OK) return 0;
    return train_layout(d).total;
}

gqe_status gqe_attn_fwd_train(const gqe_shape* s, const void* x, const void* Wr, const float* br, const void* Wq,
                              const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo, void* out,
                              int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes, void* stream) {
    return fwd_impl(s, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, idx_out, w_out, ws, ws_bytes, stream, nullptr, true);
}

gqe_status gqe_attn_fwd_train_routed(const gqe_shape* s, const void* x, const void* Wr, const float* br,
                                     const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh,
                                     const void* Wo, const int32_t* idx, void* out, float* w_out, void* ws,
                                     size_t ws_bytes, void* stream) {
    if (s != nullptr && idx == nullptr) return GQE_ERR_NULL;
    return fwd_impl(s, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, nullptr, w_out, ws, ws_bytes, stream, nullptr, true,
                    idx);
}

gqe_status gqe_attn_bwd_timed(const gqe_shape* s, const void* x, const void* Wr, const void* Wq, const void* Wk,
                              const void* Wv, const void* Wq_sh, const void* Wo, const void* dout, float aux_coef,
                              float* dx, float* dWr, float* dbr, float* dWq, float* dWk, float* dWv, float* dWq_sh,
                              float* dWo, float* aux_loss, void* ws, size_t ws_bytes, void* stream,
                              void* const* events) {
    return bwd_impl(s, x, Wr, Wq, Wk, Wv, Wq_sh, Wo, dout, aux_coef, dx, dWr, dbr, dWq, dWk, dWv, dWq_sh, dWo,
                    aux_loss, ws, ws_bytes, stream, events);
}

gqe_status gqe_attn_bwd(const gqe_shape* s, const void* x, const void* Wr, const void* Wq, const void* Wk,
                        const void* Wv, const void* Wq_sh, const void* Wo, const void* dout, float aux_coef, float* dx,
                        float* dWr, float* dbr, float* dWq, float* dWk, float* dWv, float* dWq_sh, float* dWo,
                        float* aux_loss, void* ws, size_t ws_bytes, void* stream) {
    return bwd_impl(s, x, Wr, Wq, Wk, Wv, Wq_sh, Wo, dout, aux_coef, dx, dWr, dbr, dWq, dWk, dWv, dWq_sh, dWo,
                    aux_loss, ws, ws_bytes, stream, nullptr);
}

size_t gqe_decode_workspace_bytes(const gqe_shape* s) {
    Dims c, t;
    if (check_decode(s, &c, &t) != GQE_OK) return 0;
    return decode_layout(c, t).total;
}

gqe_status gqe_decode_step(const gqe_shape* s, const int32_t* pos, const void* x, const void* Wr, const float* br,
                           const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo,
                           void* k_cache, void* vt_cache, void* out, int32_t* idx_out, float* w_out, void* ws,
                           size_t ws_bytes, void* stream) {
    return decode_impl(s, pos, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, k_cache, vt_cache, out, idx_out, w_out, ws, ws_bytes,
                       stream, nullptr);
}

gqe_status gqe_decode_step_timed(const gqe_shape* s, const int32_t* pos, const void* x, const void* Wr,
                                 const float* br, const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh,
                                 const void* Wo, void* k_cache, void* vt_cache, void* out, int32_t* idx_out,
                                 float* w_out, void* ws, size_t ws_bytes, void* stream, void* const* events) {
    return decode_impl(s, pos, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, k_cache, vt_cache, out, idx_out, w_out, ws, ws_bytes,
                       stream, events);
}

// ---------------------------------------------------------------------------
// Dense GQA baseline
// ---------------------------------------------------------------------------
static gqe_status check_gqa(int64_t B, int64_t T, int64_t D, int32_t Hq, int32_t G, int32_t d_h, int32_t dtype,
                            Dims* o) {
    if (B < 1 || T < 1 || D < 1 || Hq < 1 || G < 1) return GQE_ERR_SHAPE;
    if (Hq % G != 0 || Hq > 256) return GQE_ERR_SHAPE;
    gqe_shape s{};
    s.B = B; s.T = T; s.D = D; s.G = G; s.M = Hq / G; s.k = Hq / G; s.d_h = d_h;
    s.shared_kv_group = 0; s.dtype = dtype;
    s.variant = GQE_FULL;
    return check_shape(&s, o);
}

struct GqaWs {
    size_t Q, K, Vt, C, total;
};

static GqaWs gqa_layout(const Dims& d) {
    GqaWs L;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t a = o; o = align_up(o + bytes, 256); return a; };
    const int Hq = d.E;
    L.Q = take((size_t)d.N * Hq * d.d * d.esz);
    L.K = take((size_t)d.G * d.B * d.Tpad * d.d * d.esz);
    L.Vt = take((size_t)d.G * d.B * d.Tpad * d.d * d.esz);
    L.C = take((size_t)d.N * Hq * d.d * d.esz);
    L.total = o;
    return L;
}

size_t gqa_workspace_bytes(int64_t B, int64_t T, int64_t D, int32_t Hq, int32_t G, int32_t d_h, int32_t dtype) {
    Dims d;
    if (check_gqa(B, T, D, Hq, G, d_h, dtype, &d) != GQE_OK) return 0;
    return gqa_layout(d).total;
}

gqe_status gqa_attn_fwd_timed(int64_t B, int64_t T, int64_t D, int32_t Hq, int32_t G, int32_t d_h,
                              int32_t dtype, const void* x, const void* Wq, const void* Wk, const void* Wv,
                              const void* Wo, void* out, void* ws, size_t ws_bytes, void* stream,
                              void* const* events) {
    Dims d;
    gqe_status rc = check_gqa(B, T, D, Hq, G, d_h, dtype, &d);
    if (rc != GQE_OK) return rc;
    if (!x || !Wq || !Wk || !Wv || !Wo || !out || !ws) return GQE_ERR_NULL;
    if (!aligned16(x) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) || !aligned16(Wo) ||
        !aligned16(out) || !aligned16(ws))
        return GQE_ERR_ALIGN;
    const GqaWs L = gqa_layout(d);
    if (ws_bytes < L.total) return GQE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const int64_t qld = (int64_t)Hq * d.d;
    const Marks mk{events, st};
    mk.at(0);
    SegList sl = proj_base(d, x, d.D, d.N, (int)d.D);
    sl.add(Wk, d.G * d.d, at(ws, L.K), OUT_HEADS, 0, nullptr);
    sl.add(Wq, Hq * d.d, at(ws, L.Q), OUT_ROWS, qld, nullptr, q_scale(d));
    sl.add(Wv, d.G * d.d, at(ws, L.Vt), OUT_HEADS_T, 0, nullptr);
    run_proj(d, sl, st);
    AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.Q0 = at(ws, L.Q);
    a.q0_ld = qld;
    a.Q1 = nullptr;
    a.K = at(ws, L.K);
    a.Vt = at(ws, L.Vt);
    a.O = at(ws, L.C);
    a.o_ld = qld;
    a.R = Hq / G;              // head h reads group h / (Hq/G)
    a.kv1 = 0;
    mk.at(1);
    run_attention(d, a, st);
    mk.at(2);
    SegList so = proj_base(d, at(ws, L.C), qld, d.N, (int)qld);
    so.add(Wo, (int)d.D, out, OUT_ROWS, d.D, nullptr);
    run_proj(d, so, st);
    mk.at(3);
    return last_hip();
}

gqe_status gqa_attn_fwd(int64_t B, int64_t T, int64_t D, int32_t Hq, int32_t G, int32_t d_h, int32_t dtype,
                        const void* x, const void* Wq, const void* Wk, const void* Wv, const void* Wo, void* out,
                        void* ws, size_t ws_bytes, void* stream) {
    return gqa_attn_fwd_timed(B, T, D, Hq, G, d_h, dtype, x, Wq, Wk, Wv, Wo, out, ws, ws_bytes, stream, nullptr);
}

gqe_status gqe_mfma_probe(int64_t workgroups, int32_t iters, float* out, void* stream) {
    if (out == nullptr) return GQE_ERR_NULL;
    if (workgroups < 1 || workgroups > (int64_t)1 << 20 || iters < 1) return GQE_ERR_SHAPE;
    if (!aligned16(out)) return GQE_ERR_ALIGN;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, iters, out);
    return last_hip();
}

const char* gqe_status_str(gqe_status st) {
    switch (st) {
        case GQE_OK: return "GQE_OK: success";
        case GQE_ERR_NULL: return "GQE_ERR_NULL: a required pointer is NULL";
        case GQE_ERR_SHAPE: return "GQE_ERR_SHAPE: inconsistent or out-of-range sizes";
        case GQE_ERR_UNSUPPORTED: return "GQE_ERR_UNSUPPORTED: sizes the library does not handle";
        case GQE_ERR_WORKSPACE: return "GQE_ERR_WORKSPACE: workspace smaller than required";
        case GQE_ERR_ALIGN: return "GQE_ERR_ALIGN: a pointer is not 16-byte aligned";
        case GQE_ERR_HIP: return "GQE_ERR_HIP: the HIP runtime reported an error";
        case GQE_ERR_SCRATCH: return "GQE_ERR_SCRATCH: the shape needs more workspace than the static scratch holds";
        default: break;
    }
    return "unknown gqe_status";
}

}  // extern "C"
