// Causal flash attention over dense per-group K/V for many query heads.
//
// The GQE layer runs one attention per picked expert and one for the shared
// head ("Grouped Query Experts" explainer, technical summary, "Architecture
// and routing": every picked expert and the always-on shared head attend over
// their group's unchanged K/V; FrontiersMind GQE article, part 4). The dense
// GQA baseline runs one per query head. Both are the same kernel: a head is a
// query source (base, row stride), a KV group and an output column.
//
// Per workgroup: one head, one sequence, BQ=128 queries (4 waves x 32).
// K/V tiles of 64 keys are staged in double-buffered LDS and shared by the
// four waves. Scores are computed transposed, S^T = K Q^T, so that after the
// softmax each lane already holds, for its query column, the key slots the
// second product O^T = V^T P^T wants as its B operand: no shuffles between
// the two MFMA stages. V is kept transposed in HBM ([group][d][token]) so its
// A operand reads contiguous keys. Softmax state is fp32 and online; the
// 1/sqrt(d) scale and log2(e) fold into one FMA before v_exp_f32.
#pragma once

#include "gqe_common.hpp"

namespace gqe {

struct AttnArgs {
    const void* Q0;      // main heads: query of token n, head h at Q0 + n*q0_ld + h*d
    const void* Q1;      // extra (shared) head: Q1 + n*q1_ld, or null
    const void* K;       // [G][Bt][Tpad][d]
    const void* Vt;      // [G][d][Bt*Tpad]
    void* O;             // main head h -> O + n*o_ld + h*d; extra head -> O + n*o_ld + o1_col
    int64_t q0_ld, q1_ld, o_ld;
    int64_t T, Tpad;
    int32_t Bt;
    int32_t H0;          // number of main heads
    int32_t kv_div;      // main head h reads KV group h / kv_div
    int32_t kv1;         // KV group of the extra head
    int32_t H;           // H0 + (Q1 != null)
    int32_t n_qt;        // query tiles per sequence
    int32_t o1_col;
    float scale_log2;    // log2(e) / sqrt(d)
};

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnArgs a) {
    constexpr int BQ = 128, BKV = 64;
    constexpr int ES = sizeof(T);
    constexpr int DK = D / 32;                 // 32-wide contraction steps over d
    constexpr int CB = D / 16;                 // 16-wide blocks of the output columns
    constexpr int KP = D * ES + 16;            // LDS pitch of a K row (bytes)
    constexpr int VP = BKV * ES + 16;          // LDS pitch of a V^T row (bytes)
    constexpr int K_BYTES = BKV * KP, V_BYTES = D * VP;
    constexpr int STAGE = K_BYTES + V_BYTES;
    constexpr int KCH = D * ES / 16;           // 16-byte chunks per K row
    constexpr int VCH = BKV * ES / 16;         // 16-byte chunks per V^T row
    constexpr int K_PER_T = BKV * KCH / 256;
    constexpr int V_PER_T = D * VCH / 256;
    constexpr int VEC = 16 / ES;
    static_assert(K_PER_T >= 1 && V_PER_T >= 1, "tile must cover 256 threads");
    __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int hb = a.H * a.Bt;
    const int qt = a.n_qt - 1 - (int)(blockIdx.x / hb);     // longest rows first
    const int rem = (int)(blockIdx.x % hb);
    const int h = rem / a.Bt, b = rem % a.Bt;
    const bool extra = h >= a.H0;
    const int g = extra ? a.kv1 : h / a.kv_div;
    const T* Qh = extra ? (const T*)a.Q1 : (const T*)a.Q0 + (int64_t)h * D;
    const int64_t qld = extra ? a.q1_ld : a.q0_ld;
    T* Oh = (T*)a.O + (extra ? (int64_t)a.o1_col : (int64_t)h * D);
    const T* Kg = (const T*)a.K + ((int64_t)g * a.Bt + b) * a.Tpad * D;
    const int64_t vrow = (int64_t)a.Bt * a.Tpad;
    const T* Vg = (const T*)a.Vt + (int64_t)g * D * vrow + (int64_t)b * a.Tpad;
    const int64_t T_ = a.T;
    const int64_t tok0 = (int64_t)b * T_;

    const int q_base = qt * BQ + wave * 32;     // first query of this wave
    // Queries as the B operand of S^T = K Q^T: column l16 of block qb, d slice dk.
    Frag<T> qf[2][DK];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int t = q_base + qb * 16 + l16;
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            if (t < T_) {
                qf[qb][dk] = ld_frag<T>(Qh + (tok0 + t) * qld + dk * 32 + 8 * q4);
            } else {
                Frag<T> z;
                if constexpr (ES == 2) {
                    z.v = bf16x8{};
                } else {
                    z.lo = f32x4{0.f, 0.f, 0.f, 0.f};
                    z.hi = z.lo;
                }
                qf[qb][dk] = z;
            }
        }
    }

    f32x4 o[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[cb][0] = o[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    const float c = a.scale_log2;

    const int q_hi = (int)min<int64_t>(T_, (int64_t)qt * BQ + BQ);   // queries of the tile are < q_hi
    const int n_kv = (q_hi - 1) / BKV + 1;

    u32x4 rk[K_PER_T], rv[V_PER_T];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    auto gload = [&](int j) {
        const int s0 = j * BKV;
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            const int it = tid + 256 * i, r = it / KCH, ch = it % KCH;
            rk[i] = (s0 + r < T_) ? ld16(Kg + (int64_t)(s0 + r) * D + ch * VEC) : zero;
        }
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i) {
            const int it = tid + 256 * i, r = it / VCH, ch = it % VCH;
            const int s = s0 + ch * VEC;       // first key of this chunk (in-bounds: Tpad pads)
            u32x4 v = ld16(Vg + (int64_t)r * vrow + s);
            if (s + VEC > T_) {                 // zero the keys at or beyond T
                T* e = reinterpret_cast<T*>(&v);
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    if (s + q >= T_) e[q] = from_f32<T>(0.f);
            }
            rv[i] = v;
        }
    };
    auto sstore = [&](int buf) {
        char* Ks = lds + buf * STAGE;
        char* Vs = Ks + K_BYTES;
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            const int it = tid + 256 * i;
            st16(Ks + (it / KCH) * KP + (it % KCH) * 16, rk[i]);
        }
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i) {
            const int it = tid + 256 * i;
            st16(Vs + (it / VCH) * VP + (it % VCH) * 16, rv[i]);
        }
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int j = 0; j < n_kv; ++j) {
        if (j + 1 < n_kv) gload(j + 1);
        const int s0 = j * BKV;
        if (s0 <= q_base + 31) {               // else every key is above every query of this wave
            const char* Ks = lds + (j & 1) * STAGE;
            const char* Vs = Ks + K_BYTES;
            f32x4 s[4][2];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) s[kb][0] = s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dk = 0; dk < DK; ++dk)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const Frag<T> kf = ld_frag<T>(Ks + (kb * 16 + l16) * KP + (dk * 32 + 8 * q4) * ES);
                    s[kb][0] = mma16(kf, qf[0][dk], s[kb][0]);
                    s[kb][1] = mma16(kf, qf[1][dk], s[kb][1]);
                }
            if (s0 + BKV - 1 > q_base) {       // a key may lie above a query: causal mask
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int key = s0 + kb * 16 + 4 * q4 + v;
                            const int qry = q_base + qb * 16 + l16;
                            if (key > qry) s[kb][qb][v] = -INFINITY;
                        }
            }
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float mx = s[0][qb][0];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[kb][qb][v]);
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run[qb], mx);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float corr = __builtin_amdgcn_exp2f((m_run[qb] - m_use) * c);
                m_run[qb] = m_new;
                const float nmc = -m_use * c;
                float ls = 0.f;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][v], c, nmc));
                        s[kb][qb][v] = p;
                        ls += p;
                    }
                l_run[qb] = l_run[qb] * corr + ls;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) o[cb][qb] *= corr;
            }
            // O^T += V^T P^T, 32 keys per step: slot jj of lane group q4 is key
            // 32*kc + 4*q4 + jj (jj < 4) or 32*kc + 16 + 4*q4 + (jj - 4).
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                Frag<T> pf[2];
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
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
                }
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const char* vr = Vs + (cb * 16 + l16) * VP;
                    Frag<T> vf;
                    if constexpr (ES == 2) {
                        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr + (32 * kc + 4 * q4) * ES);
                        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + (32 * kc + 16 + 4 * q4) * ES);
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            vf.v[v] = lo[v];
                            vf.v[4 + v] = hi[v];
                        }
                    } else {
                        vf.lo = *reinterpret_cast<const f32x4*>(vr + (32 * kc + 4 * q4) * ES);
                        vf.hi = *reinterpret_cast<const f32x4*>(vr + (32 * kc + 16 + 4 * q4) * ES);
                    }
                    o[cb][0] = mma16(vf, pf[0], o[cb][0]);
                    o[cb][1] = mma16(vf, pf[1], o[cb][1]);
                }
            }
        }
        if (j + 1 < n_kv) sstore((j + 1) & 1);
        __syncthreads();
    }

    // Normalise and store: lane holds query l16 of block qb, columns cb*16 + 4*q4 + v.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float l = l_run[qb];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const float inv = 1.f / l;
        const int t = q_base + qb * 16 + l16;
        if (t >= T_) continue;
        T* orow = Oh + (tok0 + t) * a.o_ld;
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
