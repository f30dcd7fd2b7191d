// Chunked-prefill attention for sequences with two or more query tokens in
// the step.
//
// A prefill chunk is a dense contraction (vllm-metal v0.4.0 release post,
// "The same stack on DGX Spark": a long prompt is one large matmul, bound by
// compute; "Faster prefill on M5": the prefill path runs on the matrix units).
// Its QK^T and PV products run on the gfx950 matrix cores; the online softmax
// between them runs on the vector ALUs in float32.  A chunk attends to all the
// sequence's cached keys plus the chunk's own earlier tokens: query token i of
// an n-token chunk over L keys sits at position L - n + i ("How vllm-metal fits
// into vLLM": chunked prefill shares each step with decodes).
//
// Work unit: one workgroup of four wavefronts per (sequence, kv head, tile of
// query tokens).  The G query heads of the kv head are folded into the tile's
// rows (row = token * G + head), so every staged K/V page serves all of them.
// Each wavefront owns 32 rows (two 16-column MFMA tiles).  Pairs of KV pages
// (32 keys) are staged in LDS once per workgroup, double-buffered, and read by
// all four wavefronts.  The sequence that owns a tile is found by a binary
// search over query_start_loc ("Replacing attention, reusing the rest": each
// threadgroup finds its request by binary search over cu_seqlens).
#pragma once

#include "pkv_device.hpp"

namespace pkv {

struct PrefillParams {
    void* out;
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    const int32_t* qsl;
    const int32_t* kv_start;
    int num_seqs;
    int max_blocks;
    int Hq;
    int Hkv;
    int G;
    int tile_tokens;   // query tokens per workgroup: floor(128 / G)
    int max_seqlen_k;
    int64_t total_q;
    int64_t num_blocks;
    float scale_log2;
};

constexpr int kPrefillWaves = 4;
constexpr int kPrefillRows = 32 * kPrefillWaves;

template <typename T, int D>
struct PrefillGeom {
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int RB = D * EB;
    static constexpr int RS = RB + 16;
    static constexpr int PAGE_LDS = kPage * RS;
    static constexpr int STAGE = 4 * PAGE_LDS;          // K page a, K page b, V page a, V page b
    static constexpr int NT = D / 16;
    static constexpr int KCH = RB / 64;
    static constexpr int CPR = RB / 16;
    static constexpr int LCH = 4 * kPage * CPR / (kPrefillWaves * kWave);  // chunks per thread per stage
};

template <typename T, int D>
__global__ void __launch_bounds__(256) prefill_kernel(PrefillParams p) {
    using Gm = PrefillGeom<T, D>;
    constexpr bool kBF = !__is_same(T, float);
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * Gm::STAGE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int g = blockIdx.y;
    const int bid = blockIdx.x;
    const int BQ = p.tile_tokens;

    // ---- which sequence owns this tile: largest s with qsl[s]/BQ + s <= bid
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.qsl[mid] / BQ + mid <= bid) lo = mid; else hi = mid - 1;
    }
    const int s = lo;
    int q0 = p.qsl[s];
    int n = p.qsl[s + 1] - q0;
    if (q0 < 0 || q0 >= p.total_q || n < 2) return;
    if (n > p.total_q - q0) n = (int)(p.total_q - q0);
    const int qt = bid - (q0 / BQ + s);
    const int tok0 = qt * BQ;
    if (qt < 0 || tok0 >= n) return;
    const int ntok = min(BQ, n - tok0);

    const SeqRange r = seq_range(p.seq_lens, p.kv_start, s, p.max_seqlen_k, p.max_blocks);
    const int pos_min = r.L - n + tok0;           // position of the tile's first token
    const int pos_max = pos_min + ntok - 1;       // ... and of its last
    if (pos_max < r.a) {
        // every row sees no key (only with metadata outside the contract): write zeros
        for (int rr = tid; rr < ntok * p.G; rr += blockDim.x) {
            const int tok = rr / p.G, hh = rr % p.G;
            uint8_t* orow = static_cast<uint8_t*>(p.out) +
                            ((int64_t)(q0 + tok0 + tok) * p.Hq + g * p.G + hh) * Gm::RB;
            for (int c = 0; c < Gm::CPR; ++c) st16(orow + c * 16, u32x4{0, 0, 0, 0});
        }
        return;
    }
    const int first_page = r.first_page;
    const int last_page = pos_max / kPage;
    const int nstage = (last_page - first_page + 2) / 2;
    const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks;

    // ---- rows of this wavefront: two 16-column tiles
    int pos[2];
    bool rvalid[2];
    int64_t orow_idx[2];
    u32x4 qop[2][Gm::KCH];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int row = wave * 32 + nt * 16 + col;
        const int tok = row / p.G, hh = row - (row / p.G) * p.G;
        rvalid[nt] = tok < ntok;
        pos[nt] = rvalid[nt] ? pos_min + tok : -1;
        orow_idx[nt] = (int64_t)(q0 + tok0 + (rvalid[nt] ? tok : 0)) * p.Hq + g * p.G + hh;
        const uint8_t* qrow = static_cast<const uint8_t*>(p.q) + orow_idx[nt] * Gm::RB;
#pragma unroll
        for (int i = 0; i < Gm::KCH; ++i) {
            u32x4 v = ld16(qrow + i * 64 + grp * 16);
            qop[nt][i] = rvalid[nt] ? v : u32x4{0, 0, 0, 0};
        }
    }

    const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
    const uint8_t* vpool = static_cast<const uint8_t*>(p.v_pool);
    const int64_t page_stride = (int64_t)p.Hkv * kPage * Gm::RB;
    const int64_t head_off = (int64_t)g * kPage * Gm::RB;

    auto load_stage = [&](int st, u32x4 (&reg)[Gm::LCH]) {
        const int pa = first_page + 2 * st;
        const int64_t ba = safe_block(bt, pa, p.num_blocks);
        const int64_t bb = safe_block(bt, pa + 1 <= last_page ? pa + 1 : pa, p.num_blocks);
#pragma unroll
        for (int c = 0; c < Gm::LCH; ++c) {
            const int ci = c * (kPrefillWaves * kWave) + tid;
            const int buf = ci / (kPage * Gm::CPR);
            const int within = ci - buf * (kPage * Gm::CPR);
            const uint8_t* pool = (buf < 2) ? kpool : vpool;
            const int64_t blk = (buf & 1) ? bb : ba;
            reg[c] = ld16(pool + blk * page_stride + head_off + (int64_t)within * 16);
        }
    };
    auto store_stage = [&](int slot, const u32x4 (&reg)[Gm::LCH]) {
        uint8_t* base = lds + slot * Gm::STAGE;
#pragma unroll
        for (int c = 0; c < Gm::LCH; ++c) {
            const int ci = c * (kPrefillWaves * kWave) + tid;
            const int buf = ci / (kPage * Gm::CPR);
            const int within = ci - buf * (kPage * Gm::CPR);
            const int row = within / Gm::CPR, cc = within - (within / Gm::CPR) * Gm::CPR;
            st16(base + buf * Gm::PAGE_LDS + row * Gm::RS + cc * 16, reg[c]);
        }
    };

    f32x4 acc[2][Gm::NT];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int t = 0; t < Gm::NT; ++t) acc[nt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

    {
        u32x4 reg[Gm::LCH];
        load_stage(0, reg);
        store_stage(0, reg);
    }
    __syncthreads();

    for (int st = 0; st < nstage; ++st) {
        const int pa = first_page + 2 * st;
        const bool more = st + 1 < nstage;
        u32x4 reg[Gm::LCH];
        if (more) load_stage(st + 1, reg);
        const uint8_t* sb = lds + (st & 1) * Gm::STAGE;

        // ---- S^T tiles: keys of page x as rows, this wavefront's rows as columns
        f32x4 sx[2][2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            u32x4 kop[Gm::KCH];
#pragma unroll
            for (int i = 0; i < Gm::KCH; ++i)
                kop[i] = ld16(sb + x * Gm::PAGE_LDS + col * Gm::RS + i * 64 + grp * 16);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (kBF) {
#pragma unroll
                    for (int i = 0; i < Gm::KCH; ++i) sacc = mfma_bf16(kop[i], qop[nt][i], sacc);
                } else {
#pragma unroll
                    for (int i = 0; i < Gm::KCH; ++i)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            sacc = mfma_f32(__uint_as_float(kop[i][t]),
                                            __uint_as_float(qop[nt][i][t]), sacc);
                }
                sx[nt][x] = sacc;
            }
        }
        const bool edge = (pa * kPage < r.a) || (pa * kPage + 2 * kPage - 1 > pos_min);
        bool kval[8];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int key = (pa + x) * kPage + grp * 4 + t;
                kval[x * 4 + t] = !edge || (key >= r.a && key <= pos_max);
            }
        u32x4 pb[2];
        float pv[2][8];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            float sv[8];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int key = (pa + x) * kPage + grp * 4 + t;
                    const bool ok = !edge || (key >= r.a && key <= pos[nt]);
                    sv[x * 4 + t] = ok ? sx[nt][x][t] * p.scale_log2 : -INFINITY;
                }
            float mt = sv[0];
#pragma unroll
            for (int t = 1; t < 8; ++t) mt = fmaxf(mt, sv[t]);
            mt = col_max(mt);
            const float m_new = fmaxf(m_run[nt], mt);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run[nt] - m_use);
            m_run[nt] = m_new;
            float psum = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                pv[nt][t] = fast_exp2(sv[t] - m_use);
                psum += pv[nt][t];
            }
            l_run[nt] = l_run[nt] * alpha + psum;
#pragma unroll
            for (int t = 0; t < Gm::NT; ++t) acc[nt][t] *= alpha;
            if constexpr (kBF)
                pb[nt] = u32x4{pack_bf16(pv[nt][0], pv[nt][1]), pack_bf16(pv[nt][2], pv[nt][3]),
                               pack_bf16(pv[nt][4], pv[nt][5]), pack_bf16(pv[nt][6], pv[nt][7])};
        }

        // ---- O^T += V^T P^T
        if constexpr (kBF) {
            const uint16_t* l16 = reinterpret_cast<const uint16_t*>(sb + 2 * Gm::PAGE_LDS);
#pragma unroll
            for (int t = 0; t < Gm::NT; ++t) {
                const int d = t * 16 + col;
                u32x4 a;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int x = w >> 1;
                    const int k0 = grp * 4 + (w & 1) * 2;
                    const int base = (x * Gm::PAGE_LDS + k0 * Gm::RS) / 2 + d;
                    uint32_t lo16 = l16[base];
                    uint32_t hi16 = l16[base + Gm::RS / 2];
                    if (edge) {
                        lo16 = kval[2 * w] ? lo16 : 0u;
                        hi16 = kval[2 * w + 1] ? hi16 : 0u;
                    }
                    a[w] = lo16 | (hi16 << 16);
                }
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[nt][t] = mfma_bf16(a, pb[nt], acc[nt][t]);
            }
        } else {
            const float* lf = reinterpret_cast<const float*>(sb + 2 * Gm::PAGE_LDS);
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int key = grp * 4 + u;
                    const bool ok = kval[x * 4 + u];
#pragma unroll
                    for (int t = 0; t < Gm::NT; ++t) {
                        float v = lf[(x * Gm::PAGE_LDS + key * Gm::RS) / 4 + t * 16 + col];
                        v = ok ? v : 0.f;
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
                            acc[nt][t] = mfma_f32(v, pv[nt][x * 4 + u], acc[nt][t]);
                    }
                }
        }
        if (more) store_stage((st + 1) & 1, reg);
        __syncthreads();
    }

#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const float l_tot = col_sum(l_run[nt]);
        if (!rvalid[nt]) continue;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint8_t* orow = static_cast<uint8_t*>(p.out) + orow_idx[nt] * Gm::RB;
#pragma unroll
        for (int t = 0; t < Gm::NT; ++t) {
            const int d = t * 16 + grp * 4;
            if constexpr (kBF) {
                uint32_t w0 = pack_bf16(acc[nt][t][0] * inv, acc[nt][t][1] * inv);
                uint32_t w1 = pack_bf16(acc[nt][t][2] * inv, acc[nt][t][3] * inv);
                *reinterpret_cast<uint2*>(orow + d * 2) = make_uint2(w0, w1);
            } else {
                *reinterpret_cast<f32x4*>(orow + d * 4) = acc[nt][t] * inv;
            }
        }
    }
}

}  // namespace pkv
