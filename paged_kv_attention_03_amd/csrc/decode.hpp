// Split-key decode attention for sequences with one query token, and the
// merge of the per-split partial results.
//
// A decode step reads every visible key and value once and does a few flops
// per byte: it is bound by memory bandwidth (vllm-metal v0.4.0 release post,
// "The same stack on DGX Spark": decode is bandwidth-bound, prefill is
// compute-bound).  The kernel therefore streams whole KV pages with coalesced
// 16-byte loads, keeps everything else on chip, and spreads each sequence's
// keys over many workgroups (split-key) so that a handful of long sequences
// still fills the GPU; a second small kernel merges the partial results with
// the usual log-sum-exp rescaling.
//
// Work unit: one wavefront per (sequence s, kv head g, split j).  The G query
// heads that share kv head g are the 16 columns of a 16x16 matrix-core tile
// (columns >= G are zero), so one pass over a page serves all of them:
//   S^T[key][head] = K_page[key][:] . q[head][:]      (MFMA, keys as rows)
//   O^T[d][head]  += V^T[d][key] * P^T[key][head]      (MFMA, d as rows)
// K goes straight from global memory into the A-operand registers (each lane
// reads 16-byte pieces of one key row, so every load instruction touches 16
// rows x 64 contiguous bytes).  V is staged through LDS, because the PV
// product needs it key-major per lane (a transpose).  The online softmax keeps
// one running max and sum per column; the max over the four lane groups of a
// column is a two-step wavefront shuffle.  Keys outside [kv_start, seq_len)
// are masked by selection, and their V entries are zeroed before the product,
// so whatever bytes a partial or padding page holds (NaN included) never
// reaches the output.
#pragma once

#include "pkv_device.hpp"

namespace pkv {

struct DecodeParams {
    void* out;
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    const int32_t* qsl;
    const int32_t* kv_start;
    float* ws_o;    // [num_seqs][Hq][max_splits][D] unnormalised partial outputs
    float* ws_ml;   // [num_seqs][Hq][max_splits][2] (running max in log2 units, sum)
    int num_seqs;
    int max_blocks;
    int Hq;
    int Hkv;
    int G;
    int pages_per_split;
    int max_splits;
    int max_seqlen_k;
    int64_t total_q;
    int64_t num_blocks;
    float scale_log2;  // softmax scale * log2(e)
};

__device__ __forceinline__ void wave_lds_fence() {
    // Orders this wave's LDS writes before its later LDS reads (and the reverse)
    // without waiting on outstanding global loads.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

template <typename T, int D>
struct DecodeGeom {
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int RB = D * EB;                  // bytes per K/V row
    static constexpr int RS = RB + 16;                 // LDS row stride (bank spread)
    static constexpr int PAGE_LDS = kPage * RS;        // LDS bytes per staged V page
    static constexpr int NT = D / 16;                  // 16-wide d tiles of the output
    static constexpr int VCH = RB * kPage / 16 / kWave;  // 16-B chunks per lane per V page
    static constexpr int KCH = RB / 64;                // 16-B chunks per lane per K page
    static constexpr int CPR = RB / 16;                // 16-B chunks per row
};

template <typename T, int D>
__global__ void __launch_bounds__(64) decode_kernel(DecodeParams p) {
    using Gm = DecodeGeom<T, D>;
    constexpr bool kBF = !__is_same(T, float);
    __shared__ __attribute__((aligned(16))) uint8_t lds_v[2 * Gm::PAGE_LDS];

    const int lane = threadIdx.x;
    const int col = lane & 15;
    const int grp = lane >> 4;

    int bid = blockIdx.x;
    const int j = bid % p.max_splits;
    bid /= p.max_splits;
    const int g = bid % p.Hkv;
    const int s = bid / p.Hkv;
    if (s >= p.num_seqs) return;
    const int q0 = p.qsl[s];
    const int qn = p.qsl[s + 1] - q0;
    if (qn != 1 || q0 < 0 || q0 >= p.total_q) return;

    const SeqRange r = seq_range(p.seq_lens, p.kv_start, s, p.max_seqlen_k, p.max_blocks);
    const int npages = r.end_page - r.first_page;
    const int P = p.pages_per_split;
    const int nsplit = npages > 0 ? (npages + P - 1) / P : 1;
    if (j >= nsplit) return;
    const int pg_lo = r.first_page + j * P;
    const int pg_hi = min(pg_lo + P, r.end_page);
    const int kv_lo = max(r.a, pg_lo * kPage);
    const int kv_hi = min(r.L, pg_hi * kPage);
    const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks;
    const int h = g * p.G + col;
    const bool hvalid = col < p.G;

    const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
    const uint8_t* vpool = static_cast<const uint8_t*>(p.v_pool);
    const int64_t page_stride = (int64_t)p.Hkv * kPage * Gm::RB;  // bytes per physical page
    const int64_t head_off = (int64_t)g * kPage * Gm::RB;

    // ---- query operand (B of S^T = K q^T): column `col`, k-slots of group `grp`
    u32x4 qop[Gm::KCH];
    {
        const uint8_t* qrow = static_cast<const uint8_t*>(p.q) +
                              ((int64_t)q0 * p.Hq + (hvalid ? h : 0)) * Gm::RB;
#pragma unroll
        for (int i = 0; i < Gm::KCH; ++i) {
            u32x4 v = ld16(qrow + i * 64 + grp * 16);
            qop[i] = hvalid ? v : u32x4{0, 0, 0, 0};
        }
    }

    f32x4 acc[Gm::NT];
#pragma unroll
    for (int t = 0; t < Gm::NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // Pages are processed two at a time (32 keys = one bf16 MFMA depth).
    const int npair = (pg_hi - pg_lo + 1) / 2;
    u32x4 kc[2][Gm::KCH], vc[2][Gm::VCH];
    auto load_pair = [&](int pa, u32x4 (&kr)[2][Gm::KCH], u32x4 (&vr)[2][Gm::VCH]) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int pg = (pa + x < pg_hi) ? pa + x : pa;
            const int64_t blk = safe_block(bt, pg, p.num_blocks);
            const uint8_t* kb = kpool + blk * page_stride + head_off;
            const uint8_t* vb = vpool + blk * page_stride + head_off;
#pragma unroll
            for (int i = 0; i < Gm::KCH; ++i) kr[x][i] = ld16(kb + col * Gm::RB + i * 64 + grp * 16);
#pragma unroll
            for (int c = 0; c < Gm::VCH; ++c) vr[x][c] = ld16(vb + (c * kWave + lane) * 16);
        }
    };
    auto stage_v = [&](const u32x4 (&vr)[2][Gm::VCH]) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int c = 0; c < Gm::VCH; ++c) {
                const int ci = c * kWave + lane;
                const int row = ci / Gm::CPR, cc = ci % Gm::CPR;
                st16(lds_v + x * Gm::PAGE_LDS + row * Gm::RS + cc * 16, vr[x][c]);
            }
    };

    if (npair > 0) {
        load_pair(pg_lo, kc, vc);
        stage_v(vc);
    }
    for (int it = 0; it < npair; ++it) {
        const int pa = pg_lo + 2 * it;
        const bool more = it + 1 < npair;
        u32x4 kn[2][Gm::KCH], vn[2][Gm::VCH];
        if (more) load_pair(pa + 2, kn, vn);
        wave_lds_fence();

        // ---- logits for 2 pages: lane holds keys 4*grp+{0..3} of each page, column col
        f32x4 sx[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (kBF) {
#pragma unroll
                for (int i = 0; i < Gm::KCH; ++i) sacc = mfma_bf16(kc[x][i], qop[i], sacc);
            } else {
#pragma unroll
                for (int i = 0; i < Gm::KCH; ++i)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        sacc = mfma_f32(__uint_as_float(kc[x][i][t]), __uint_as_float(qop[i][t]),
                                        sacc);
            }
            sx[x] = sacc;
        }
        const bool edge = (pa * kPage < kv_lo) || ((pa + 2) * kPage > kv_hi);
        float sv[8];
        bool valid[8];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int key = (pa + x) * kPage + grp * 4 + t;
                valid[x * 4 + t] = !edge || (key >= kv_lo && key < kv_hi);
                sv[x * 4 + t] = valid[x * 4 + t] ? sx[x][t] * p.scale_log2 : -INFINITY;
            }
        float mt = sv[0];
#pragma unroll
        for (int t = 1; t < 8; ++t) mt = fmaxf(mt, sv[t]);
        mt = col_max(mt);
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float pv[8];
        float psum = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            pv[t] = fast_exp2(sv[t] - m_use);
            psum += pv[t];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int t = 0; t < Gm::NT; ++t) acc[t] *= alpha;

        // ---- O^T += V^T P^T, V^T gathered from the staged pages
        if constexpr (kBF) {
            u32x4 pb = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]),
                        pack_bf16(pv[4], pv[5]), pack_bf16(pv[6], pv[7])};
            const uint16_t* l16 = reinterpret_cast<const uint16_t*>(lds_v);
#pragma unroll
            for (int t = 0; t < Gm::NT; ++t) {
                const int d = t * 16 + col;
                u32x4 a;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int x = w >> 1;
                    const int k0 = grp * 4 + (w & 1) * 2;
                    const int base = (x * Gm::PAGE_LDS + k0 * Gm::RS) / 2 + d;
                    uint32_t lo = l16[base];
                    uint32_t hi = l16[base + Gm::RS / 2];
                    if (edge) {
                        lo = valid[2 * w] ? lo : 0u;
                        hi = valid[2 * w + 1] ? hi : 0u;
                    }
                    a[w] = lo | (hi << 16);
                }
                acc[t] = mfma_bf16(a, pb, acc[t]);
            }
        } else {
            const float* lf = reinterpret_cast<const float*>(lds_v);
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int key = grp * 4 + u;
                    const bool ok = valid[x * 4 + u];
#pragma unroll
                    for (int t = 0; t < Gm::NT; ++t) {
                        float v = lf[(x * Gm::PAGE_LDS + key * Gm::RS) / 4 + t * 16 + col];
                        v = ok ? v : 0.f;
                        acc[t] = mfma_f32(v, pv[x * 4 + u], acc[t]);
                    }
                }
        }
        wave_lds_fence();
        if (more) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
#pragma unroll
                for (int i = 0; i < Gm::KCH; ++i) kc[x][i] = kn[x][i];
#pragma unroll
                for (int c = 0; c < Gm::VCH; ++c) vc[x][c] = vn[x][c];
            }
            stage_v(vc);
        }
    }

    const float l_tot = col_sum(l_run);
    if (!hvalid) return;
    if (nsplit == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint8_t* orow = static_cast<uint8_t*>(p.out) + ((int64_t)q0 * p.Hq + h) * Gm::RB;
#pragma unroll
        for (int t = 0; t < Gm::NT; ++t) {
            const int d = t * 16 + grp * 4;
            if constexpr (kBF) {
                uint32_t w0 = pack_bf16(acc[t][0] * inv, acc[t][1] * inv);
                uint32_t w1 = pack_bf16(acc[t][2] * inv, acc[t][3] * inv);
                *reinterpret_cast<uint2*>(orow + d * 2) = make_uint2(w0, w1);
            } else {
                *reinterpret_cast<f32x4*>(orow + d * 4) = acc[t] * inv;
            }
        }
    } else {
        const int64_t slot = ((int64_t)s * p.Hq + h) * p.max_splits + j;
        float* o = p.ws_o + slot * D;
#pragma unroll
        for (int t = 0; t < Gm::NT; ++t)
            *reinterpret_cast<f32x4*>(o + t * 16 + grp * 4) = acc[t];
        if (grp == 0) {
            p.ws_ml[slot * 2] = m_run;
            p.ws_ml[slot * 2 + 1] = l_tot;
        }
    }
}

struct MergeParams {
    void* out;
    const float* ws_o;
    const float* ws_ml;
    const int32_t* seq_lens;
    const int32_t* qsl;
    const int32_t* kv_start;
    int num_seqs;
    int max_blocks;
    int Hq;
    int pages_per_split;
    int max_splits;
    int max_seqlen_k;
    int64_t total_q;
};

// One wavefront per (sequence, query head): out = sum_j 2^(m_j - M) o_j /
// sum_j 2^(m_j - M) l_j, rounded to the output type.
template <typename T, int D>
__global__ void __launch_bounds__(64) merge_kernel(MergeParams p) {
    constexpr bool kBF = !__is_same(T, float);
    const int h = blockIdx.x % p.Hq;
    const int s = blockIdx.x / p.Hq;
    if (s >= p.num_seqs) return;
    const int q0 = p.qsl[s];
    if (p.qsl[s + 1] - q0 != 1 || q0 < 0 || q0 >= p.total_q) return;
    const SeqRange r = seq_range(p.seq_lens, p.kv_start, s, p.max_seqlen_k, p.max_blocks);
    const int npages = r.end_page - r.first_page;
    const int nsplit = npages > 0 ? (npages + p.pages_per_split - 1) / p.pages_per_split : 1;
    if (nsplit <= 1) return;
    const int64_t base = ((int64_t)s * p.Hq + h) * p.max_splits;
    float M = -INFINITY;
    for (int j = 0; j < nsplit; ++j) M = fmaxf(M, p.ws_ml[(base + j) * 2]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    constexpr int PER = D / kWave;  // output elements per lane (1 or 2)
    float num[PER], den = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] = 0.f;
    for (int j = 0; j < nsplit; ++j) {
        const float w = fast_exp2(p.ws_ml[(base + j) * 2] - Mu);
        den += w * p.ws_ml[(base + j) * 2 + 1];
        const float* o = p.ws_o + (base + j) * D;
#pragma unroll
        for (int e = 0; e < PER; ++e) num[e] += w * o[threadIdx.x * PER + e];
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    uint8_t* orow = static_cast<uint8_t*>(p.out) +
                    ((int64_t)q0 * p.Hq + h) * (int64_t)D * Elem<T>::kBytes;
    if constexpr (kBF) {
        if constexpr (PER == 2) {
            reinterpret_cast<uint32_t*>(orow)[threadIdx.x] = pack_bf16(num[0] * inv, num[1] * inv);
        } else {
            bf16x2 v = {(__bf16)(num[0] * inv), (__bf16)0.f};
            reinterpret_cast<uint16_t*>(orow)[threadIdx.x] =
                (uint16_t)(__builtin_bit_cast(uint32_t, v) & 0xffffu);
        }
    } else {
#pragma unroll
        for (int e = 0; e < PER; ++e)
            reinterpret_cast<float*>(orow)[threadIdx.x * PER + e] = num[e] * inv;
    }
}

}  // namespace pkv
