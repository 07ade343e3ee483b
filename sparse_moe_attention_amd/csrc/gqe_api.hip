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

#include "../../include/gqe.h"
#include "attention.hpp"
#include "gemm.hpp"
#include "route.hpp"

using namespace gqe;

namespace {

#ifndef GQE_PROJ_BM
#define GQE_PROJ_BM 128
#define GQE_PROJ_WM 2
#endif
using ProjBf16 = TileCfg<bf16, GQE_PROJ_BM, 128, GQE_PROJ_WM, 2>;
using ProjF32 = TileCfg<float, 128, 128, 2, 2>;
using GrpBf16 = TileCfg<bf16, 128, 64, 4, 1>;
using GrpF32 = TileCfg<float, 128, 64, 4, 1>;

constexpr int kAttnWaves = kAttnNW;             // waves per attention workgroup
constexpr int kBQ = kAttnWaves * kAttnQW;       // attention query tile
constexpr int kKVPad = kAttnBKV;  // sequence padding of the K / V^T buffers: whole key tiles

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
    // Eight resident waves per CU (two per SIMD: the register budget), in
    // whole XCD rounds.
    const int64_t tiles = n_m * a.n_tiles_n;
    const int per_cu = 8 / (Cfg::WM * Cfg::WN);
    const int64_t grid = std::min<int64_t>(tiles, per_cu * (int64_t)align_up((size_t)device_cus(), 8));
    hipLaunchKernelGGL((proj_gemm_kernel<T, Cfg>), dim3((unsigned)grid), dim3(Cfg::NTH), 0, st, a);
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
    if (d.f32) hipLaunchKernelGGL((grouped_q_kernel<float, GrpF32>), grid, dim3(GrpF32::NTH), 0, st, g);
    else hipLaunchKernelGGL((grouped_q_kernel<bf16, GrpBf16>), grid, dim3(GrpBf16::NTH), 0, st, g);
}

void run_attention(const Dims& d, AttnArgs& a, hipStream_t st) {
    a.T = d.T;
    a.Tpad = d.Tpad;
    a.Bt = (int)d.B;
    const bool xcls = a.Q1 != nullptr;
    a.n_o = (int)((d.T * a.R + kBQ - 1) / kBQ);
    a.n_x = xcls ? (int)((d.T * (a.R + 1) + kBQ - 1) / kBQ) : 0;
    a.G = d.G;
    const int64_t n_wg = d.B * ((int64_t)(xcls ? d.G - 1 : d.G) * a.n_o + a.n_x);
    const dim3 grid((unsigned)n_wg), block(kAttnWaves * 64);
    if (d.f32) {
        if (d.d == 64) hipLaunchKernelGGL((attn_fwd_kernel<float, 64, kAttnWaves>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attn_fwd_kernel<float, 32, kAttnWaves>), grid, block, 0, st, a);
    } else {
        if (d.d == 64) hipLaunchKernelGGL((attn_fwd_kernel<bf16, 64, kAttnWaves>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attn_fwd_kernel<bf16, 32, kAttnWaves>), grid, block, 0, st, a);
    }
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
                           bool project_kv, const Marks& mk) {
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
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)d.nC), dim3(256), 0, st, idx, (const int32_t*)cbase,
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

}  // namespace

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
    hipLaunchKernelGGL((route_kernel<0>), dim3((unsigned)d.nC), dim3(256), 0, st, (const float*)lg, idx, w, hist,
                       d.N, d.G, d.M, d.k, (int)(d.variant != GQE_WEIGHTED_CONCAT));
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
    hipLaunchKernelGGL((route_kernel<1>), dim3((unsigned)d.nC), dim3(256), 0, st, (const float*)nullptr,
                       const_cast<int32_t*>(idx), (float*)nullptr, (int32_t*)at(ws, L.hist), d.N, d.G, d.M, d.k, 1);
    void* C = slots_out ? slots_out : at(ws, L.C);
    return run_post_router(d, L, ws, x, Wq, Wk, Wv, Wq_sh, Wo, idx, w, out, C, st, true, Marks{nullptr, st});
}

gqe_status gqe_attn_fwd_timed(const gqe_shape* s, const void* x, const void* Wr, const float* br,
                              const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo,
                              void* out, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes, void* stream,
                              void* const* events) {
    Dims d;
    gqe_status rc = check_shape(s, &d);
    if (rc != GQE_OK) return rc;
    if (!x || !Wr || !Wq || !Wk || !Wv || !Wq_sh || !Wo || !out || !ws) return GQE_ERR_NULL;
    if (!aligned16(x) || !aligned16(Wr) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) ||
        !aligned16(Wq_sh) || !aligned16(Wo) || !aligned16(out) || !aligned16(ws) || (br && !aligned16(br)) ||
        (idx_out && !aligned16(idx_out)) || (w_out && !aligned16(w_out)))
        return GQE_ERR_ALIGN;
    const GqeWs L = gqe_layout(d);
    if (ws_bytes < L.total) return GQE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    int32_t* idx = idx_out ? idx_out : (int32_t*)at(ws, L.idx);
    float* w = w_out ? w_out : (float*)at(ws, L.w);
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
    hipLaunchKernelGGL((route_kernel<0>), dim3((unsigned)d.nC), dim3(256), 0, st, (const float*)lg, idx, w,
                       (int32_t*)at(ws, L.hist), d.N, d.G, d.M, d.k, (int)(d.variant != GQE_WEIGHTED_CONCAT));
    return run_post_router(d, L, ws, x, Wq, Wk, Wv, Wq_sh, Wo, idx, w, out, at(ws, L.C), st, false, mk);
}

gqe_status gqe_attn_fwd(const gqe_shape* s, const void* x, const void* Wr, const float* br, const void* Wq,
                        const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo, void* out,
                        int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes, void* stream) {
    return gqe_attn_fwd_timed(s, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, idx_out, w_out, ws, ws_bytes, stream,
                              nullptr);
}

// ---------------------------------------------------------------------------
// Dense GQA baseline
// ---------------------------------------------------------------------------
static gqe_status check_gqa(int64_t B, int64_t T, int64_t D, int32_t Hq, int32_t G, int32_t d_h, int32_t dtype,
                            Dims* o) {
    if (B < 1 || T < 1 || D < 1 || Hq < 1 || G < 1) return GQE_ERR_SHAPE;
    if (Hq % G != 0 || Hq > 256) return GQE_ERR_SHAPE;
    gqe_shape s;
    s.B = B; s.T = T; s.D = D; s.G = G; s.M = Hq / G; s.k = Hq / G; s.d_h = d_h;
    s.shared_kv_group = 0; s.dtype = dtype;
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

const char* gqe_status_str(gqe_status st) {
    switch (st) {
        case GQE_OK: return "GQE_OK: success";
        case GQE_ERR_NULL: return "GQE_ERR_NULL: a required pointer is NULL";
        case GQE_ERR_SHAPE: return "GQE_ERR_SHAPE: inconsistent or out-of-range sizes";
        case GQE_ERR_UNSUPPORTED: return "GQE_ERR_UNSUPPORTED: sizes this build does not handle";
        case GQE_ERR_WORKSPACE: return "GQE_ERR_WORKSPACE: workspace smaller than required";
        case GQE_ERR_ALIGN: return "GQE_ERR_ALIGN: a pointer is not 16-byte aligned";
        case GQE_ERR_HIP: return "GQE_ERR_HIP: the HIP runtime reported an error";
    }
    return "unknown gqe_status";
}

}  // extern "C"
