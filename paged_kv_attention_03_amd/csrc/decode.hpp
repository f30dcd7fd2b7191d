// Split-key decode attention for sequences with a few query tokens (one for a
// plain decode, k + 1 for a speculative-verify window of k draft tokens), and
// the merge of the per-split partial results.
//
// A decode step reads every visible key and value once and does a few flops
// per byte: it is bound by memory bandwidth (vllm-metal v0.4.0 release post,
// "The same stack on DGX Spark": decode is bandwidth-bound, prefill is
// compute-bound).  The kernels therefore stream whole KV pages with coalesced
// 16-byte loads and keep everything else on chip.
//
// Work split (split-key, balanced): the page pairs of every decode sequence
// are counted and the list of all (kv head, sequence, page pair) units is cut
// into kDecodeWaves equal contiguous ranges -- by every wave for itself up to
// kInlinePlanSeqs sequences, by a one-workgroup plan kernel beyond.  One
// persistent wavefront streams each range, crossing from one (sequence, kv
// head) segment to the next without leaving the kernel, so every wave does
// the same number of page pairs whatever the length mix.  Wave numbers count
// along each XCD, so an XCD streams one kv head's pages (or a contiguous run
// of heads) and pages shared by several sequences are re-read from its L2.  A
// segment that lies inside one wave's range is finished there and written to
// the output; a segment cut by a range boundary leaves at most two partial
// results per wave, which a small merge kernel combines with the usual
// log-sum-exp rescaling.  Steps whose segments are all short run instead one
// wave per segment: nothing is cut and no merge follows.
//
// Per page pair, the query rows that share kv head g -- the G heads of each of
// the sequence's n query tokens, column = token * G + head, G * n <= 16 -- are
// the 16 columns of a 16x16 matrix-core tile (unused columns are zero), so one
// pass over a page serves all of them:
//   S^T[key][head] = K_page[key][:] . q[head][:]      (MFMA, keys as rows)
//   O^T[d][head]  += V^T[d][key] * P^T[key][head]      (MFMA, d as rows)
// K goes straight from global memory into the A-operand registers (each lane
// reads 16-byte pieces of one key row, so every load instruction touches 16
// rows x 64 contiguous bytes).  V is staged through LDS and read back by the
// transposing LDS read, because the PV product needs it key-major per lane
// (a transpose).  The online softmax keeps
// one running max and sum per column; the max over the four lane groups of a
// column is a two-step wavefront shuffle.  Keys outside [kv_start, seq_len)
// are masked by selection, and their V entries are zeroed before the product,
// so whatever bytes a partial or padding page holds (NaN included) never
// reaches the output.  Inside a window, token i of n sits at position
// seq_len - n + i and sees keys up to its own position: a per-column cap that
// only the last page pair of a segment can reach ("How vllm-metal fits into
// vLLM": a packed step mixes prefill chunks, decode tokens and speculative
// verify windows).
#pragma once

#include <type_traits>

#include "pkv_device.hpp"

namespace pkv {

constexpr int kDecodeWaves = 1024;     // persistent decode waves (4 per CU on 256 CUs;
                                       // measured 1-5% faster than 8 per CU)
constexpr int kPlanThreads = 1024;
constexpr int kMaxDecodeSeqs = 16384;  // sequences the plan kernel can hold in LDS
constexpr int kWindowPages = 256;      // block-table entries staged per window
constexpr int kInlinePlanSeqs = 512;   // up to this many sequences each decode wave
                                       // plans its own pieces (no plan kernel)
// Decode K/V are read with non-temporal loads.  Within a call every page of a
// (sequence, kv head) is read once, and a page several sequences share is
// re-read from the XCD's L2 shortly after its first read, which the hint
// leaves intact (an 8192-key prefix shared by 16 decodes: 0.0770 against
// 0.0768 ms with cacheable loads).  Across calls, a model with many layers
// reads every other layer's K/V and weights between two calls of one layer,
// so nothing of the previous call is left in the 256 MB Infinity Cache to
// reuse; the hint then only keeps streamed pages from displacing each other.
// Measured on MI355X with the caches cleared before each call: a pure stream
// 7.0 against 6.4 TB/s, the 16-sequence decode step 0.041 against 0.042-0.044
// ms, the mixed chunked-prefill step 0.153 against 0.160 ms.  Only a loop that
// re-runs one layer's call back to back loses (the 16-sequence agent loop:
// 0.056 against 0.052 ms), as its previous call's pages no longer stay cached.

// A wave's piece of one (sequence, kv head) segment: page pairs [pi0, pi1).
struct Portion {
    int32_t s, g, pi0, pi1;
    int32_t slot;          // -1: the whole segment is here, write the output;
                           // else partial slot (wave * 2 + 0 first / 1 last piece)
    int32_t q0;            // first query row of the sequence
    int32_t kv_lo, kv_hi;  // keys [kv_lo, kv_hi); token i of nq sees up to kv_hi - nq + i
    int32_t nq;            // query tokens of the sequence (1 <= nq <= wmax)
};

struct PlanParams {
    const int32_t* seq_lens;
    const int32_t* qsl;
    const int32_t* kv_start;
    int num_seqs;
    int Hkv;
    int max_seqlen_k;
    int max_blocks;
    int wmax;                // sequences with 1..wmax query tokens take this path
    int64_t total_q;
    int32_t* pair_prefix;    // [num_seqs + 1] page pairs of sequences before s
    int32_t* portion_begin;  // [kDecodeWaves + 1]
    Portion* portions;       // [kDecodeWaves + num_seqs * Hkv]
};

struct DecodeParams {
    void* out;
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_tables;
    const int32_t* portion_begin;  // plan-kernel mode only
    const Portion* portions;       // plan-kernel mode only
    // inline-plan mode (num_seqs <= kInlinePlanSeqs): every wave derives its
    // pieces from the step metadata; wave 0 also writes pair_prefix
    int inline_plan;
    // inline-plan mode only: wave w (= workgroup w, num_seqs * Hkv of them)
    // takes the whole segment of kv head w / num_seqs and sequence
    // w % num_seqs instead of an even share of the units, so no segment is
    // cut and no merge follows (steps whose segments are all short)
    int whole_segments;
    const int32_t* seq_lens;
    const int32_t* qsl;
    const int32_t* kv_start;
    int num_seqs;
    int max_seqlen_k;
    int wmax;
    int64_t total_q;
    int32_t* pair_prefix;
    float* ws_o;    // [kDecodeWaves * 2][ncol][D] unnormalised partial outputs
    float* ws_ml;   // [kDecodeWaves * 2][ncol][2] (running max in log2 units, sum)
    int max_blocks;
    int Hq;
    int Hkv;
    int G;
    int gmagic;     // ceil(2^16 / G): col / G == (col * gmagic) >> 16 for col < 16
    int ncol;       // G * wmax columns per partial slot
    int64_t num_blocks;
    float scale_log2;  // softmax scale * log2(e)
    // Steps whose sequences share prefixes (null otherwise): per sequence, the
    // softmax state of its shared prefix in `state` -- x: its state row (per
    // query head; x < 0: none).  The first piece of each of the sequence's
    // segments starts from it (the decode pass itself reads only the keys
    // after the prefix).
    const int4* prefix_states;
    const float* state;  // [state_rows][Hq][kStateStride]
    int64_t state_rows;
};

struct MergeParams {
    void* out;
    const float* ws_o;
    const float* ws_ml;
    const int32_t* pair_prefix;
    const int32_t* qsl;
    int num_seqs;
    int Hq;
    int Hkv;
    int G;
    int ncol;
};

// Start of wave w's unit range, and the wave whose range holds unit u.
__device__ __forceinline__ int64_t wave_start(int64_t w, int64_t U) { return w * U / kDecodeWaves; }
__device__ __forceinline__ int64_t wave_of(int64_t u, int64_t U) {
    return ((u + 1) * kDecodeWaves + U - 1) / U - 1;
}

// Units are ordered kv head first: head g's segments, one per decode sequence
// in sequence order, fill [g * P[S], (g + 1) * P[S]) where P is the exclusive
// prefix of the sequences' page pairs.  Segment (s, g) starts at:
__device__ __forceinline__ int64_t segment_start(int g, int32_t P_s, int32_t P_S) {
    return (int64_t)g * P_S + P_s;
}

// Workgroups are dealt to the 8 XCDs in turn (workgroup b runs on XCD b % 8);
// decode wave numbers count along each XCD instead, so that XCD x streams a
// contiguous eighth of the units: with the head-first order, the pages of one
// kv head (or of a contiguous run of heads).  Pages several sequences share (a
// common prefix) are then fetched once into that XCD's L2 and re-read there.
constexpr int kXcds = 8;
static_assert(kDecodeWaves % kXcds == 0, "waves spread evenly over the XCDs");
__device__ __forceinline__ int decode_wave_id() {
    return (int)(blockIdx.x % kXcds) * (kDecodeWaves / kXcds) + (int)(blockIdx.x / kXcds);
}

__device__ __forceinline__ void wave_lds_fence() {
    // Orders this wave's LDS writes before its later LDS reads (and the reverse)
    // without waiting on outstanding global loads.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Page pairs a sequence contributes to the decode path: its visible pages
// [first_page, end_page) in pairs, if it has 1..wmax query tokens, else 0.
__device__ __forceinline__ int decode_pairs(const int32_t* qsl, const int32_t* seq_lens,
                                            const int32_t* kv_start, int s, int wmax,
                                            int64_t total_q, int max_seqlen_k, int max_blocks) {
    const int q0 = qsl[s];
    const int nq = qsl[s + 1] - q0;
    const bool dec = nq >= 1 && nq <= wmax && q0 >= 0 && q0 <= total_q - nq;
    const SeqRange r = seq_range(seq_lens, kv_start, s, max_seqlen_k, max_blocks);
    return dec ? (r.end_page - r.first_page + 1) / 2 : 0;
}

// In-place exclusive scan of a[0..n) by a 1024-thread block; a[n] = total.
__device__ void block_exclusive_scan(int32_t* a, int n, int32_t* tmp) {
    const int t = threadIdx.x;
    const int per = (n + kPlanThreads - 1) / kPlanThreads;
    const int lo = min(n, t * per), hi = min(n, lo + per);
    int32_t sum = 0;
    for (int i = lo; i < hi; ++i) sum += a[i];
    tmp[t] = sum;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const int32_t v = t >= off ? tmp[t - off] : 0;
        __syncthreads();
        tmp[t] += v;
        __syncthreads();
    }
    int32_t run = tmp[t] - sum;  // exclusive prefix of this thread's chunk
    for (int i = lo; i < hi; ++i) {
        const int32_t c = a[i];
        a[i] = run;
        run += c;
    }
    if (t == kPlanThreads - 1) a[n] = tmp[t];
    __syncthreads();
}

// One workgroup: page pairs per decode sequence, their prefix, and every
// wave's list of segment pieces.
__global__ void __launch_bounds__(kPlanThreads) decode_plan_kernel(PlanParams p) {
    __shared__ int32_t C[kMaxDecodeSeqs + 1];
    __shared__ int32_t wcnt[kDecodeWaves + 1];
    __shared__ int32_t tmp[kPlanThreads];
    const int t = threadIdx.x;
    const int S = p.num_seqs;
    for (int s = t; s < S; s += kPlanThreads)
        C[s] = decode_pairs(p.qsl, p.seq_lens, p.kv_start, s, p.wmax, p.total_q, p.max_seqlen_k,
                            p.max_blocks);
    __syncthreads();
    block_exclusive_scan(C, S, tmp);
    const int64_t U = (int64_t)p.Hkv * C[S];

    // Walks the segments that intersect wave w's range; emit=false only counts.
    auto walk = [&](int w, bool emit, int32_t out_at) -> int {
        const int64_t u0 = wave_start(w, U), u1 = wave_start(w + 1, U);
        if (u0 >= u1) return 0;
        int g = (int)(u0 / C[S]);
        const int64_t r0 = u0 - (int64_t)g * C[S];
        int lo = 0, hi = S - 1;  // largest s with C[s] <= r0 (then C[s+1] > C[s])
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (C[mid] <= r0) lo = mid; else hi = mid - 1;
        }
        int s = lo;
        int64_t c = C[s + 1] - C[s];
        int count = 0;
        while (true) {
            const int64_t seg0 = segment_start(g, C[s], C[S]);
            const int64_t seg1 = seg0 + c;
            if (emit) {
                Portion q;
                q.s = s;
                q.g = g;
                q.pi0 = (int32_t)(max(u0, seg0) - seg0);
                q.pi1 = (int32_t)(min(u1, seg1) - seg0);
                q.slot = (seg0 >= u0 && seg1 <= u1) ? -1 : w * 2 + (count == 0 ? 0 : 1);
                q.q0 = p.qsl[s];
                q.nq = p.qsl[s + 1] - q.q0;
                const SeqRange r = seq_range(p.seq_lens, p.kv_start, s, p.max_seqlen_k, p.max_blocks);
                q.kv_lo = r.a;
                q.kv_hi = r.L;
                p.portions[out_at + count] = q;
            }
            ++count;
            if (seg1 >= u1) break;
            // next segment: the next sequence with pairs, else the next head's first
            do { ++s; } while (s < S && C[s + 1] == C[s]);
            if (s == S) {
                ++g;
                s = 0;
                while (C[s + 1] == C[s]) ++s;
            }
            c = C[s + 1] - C[s];
        }
        return count;
    };

    for (int w = t; w < kDecodeWaves; w += kPlanThreads) wcnt[w] = walk(w, false, 0);
    __syncthreads();
    block_exclusive_scan(wcnt, kDecodeWaves, tmp);
    for (int w = t; w < kDecodeWaves; w += kPlanThreads) walk(w, true, wcnt[w]);
    for (int w = t; w <= kDecodeWaves; w += kPlanThreads) p.portion_begin[w] = wcnt[w];
    for (int s = t; s <= S; s += kPlanThreads) p.pair_prefix[s] = C[s];
}

template <typename T, int D>
struct DecodeGeom {
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int RB = D * EB;                  // bytes per K/V row
    // LDS row stride of a staged V page.  bfloat16 pages are read by the
    // transposing read (16 lanes take 8 bytes from each of 4 consecutive
    // rows): a 32-byte pad puts those 4 rows on distinct banks.  float32
    // pages are read 4 bytes per lane, for which 16 bytes spread the rows.
    static constexpr int RS = RB + (EB == 2 ? 32 : 16);
    static constexpr int PAGE_LDS = kPage * RS;        // LDS bytes per staged V page
    static constexpr int NT = D / 16;                  // 16-wide d tiles of the output
    static constexpr int VCH = RB * kPage / 16 / kWave;  // 16-B chunks per lane per V page
    static constexpr int KCH = RB / 64;                // 16-B chunks per lane per K page
    static constexpr int CPR = RB / 16;                // 16-B chunks per row
};

// Registers of one pair of pages in flight: K in A-operand layout, V as
// loaded (16-byte chunks of the row-major page).
template <typename T, int D>
struct PairRegs {
    u32x4 k[2][DecodeGeom<T, D>::KCH];
    u32x4 v[2][DecodeGeom<T, D>::VCH];
};

// LDS of one decode wave.
template <typename T, int D>
struct DecodeLds {
    __attribute__((aligned(16))) uint8_t v[2 * DecodeGeom<T, D>::PAGE_LDS];  // staged V pages
    int32_t bid[kWindowPages];         // a window of the block-table row
    Portion port[kWave];               // this batch's segment pieces
    int32_t pref[kInlinePlanSeqs + 1]; // inline plan: page pairs before each sequence
};

// Decode wave number w of kDecodeWaves: streams its range of units with the
// LDS `L` of its own.  PS: the step has shared-prefix states to start from (a
// separate instantiation, so that plain steps run without that code).  Runs
// as a one-wave workgroup of decode_kernel, or as one wave of a workgroup of
// the single-launch step kernel.
template <typename T, int D, bool PS>
__device__ __forceinline__ void decode_wave(const DecodeParams& p, const int w, DecodeLds<T, D>& L) {
    using Gm = DecodeGeom<T, D>;
    constexpr bool kBF = !__is_same(T, float);
    uint8_t* const lds_v = L.v;
    int32_t* const lds_bid = L.bid;
    Portion* const lds_port = L.port;
    int32_t* const lds_pref = L.pref;

    const int lane = threadIdx.x & (kWave - 1);
    const int col = lane & 15;
    const int grp = lane >> 4;
    const bool inl = p.inline_plan != 0;
    const int S = p.num_seqs;
    int pb = 0, pe = 0;       // plan-kernel mode: this wave's pieces
    int64_t u0 = 0, u1 = 0;   // inline mode: this wave's units [u0, u1)
    // The waves of an XCD first touch the block table together, one cache
    // line per lane (tables up to 1 MiB), while the step metadata is read, so
    // that the block-id reads that follow the plan hit that XCD's L2 rather
    // than HBM.  The value is kept only so that the load stays.
    int bt_touch = 0;
    {
        const int local = p.whole_segments ? (w >> 3) : (w & (kDecodeWaves / kXcds - 1));
        const int64_t idx = ((int64_t)local * kWave + lane) * 32;
        if (idx < (int64_t)S * p.max_blocks) bt_touch = p.block_tables[idx];
    }
    // One wave per segment: the wave's segment, (sequence w % S, kv head
    // w / S), is its whole range, so it needs that sequence's metadata only,
    // not the plan over every sequence, and the first window of the
    // sequence's block-table row loads beside that metadata rather than after
    // it (pages 0 .. kWindowPages - 1; staged again past them as usual).  The
    // pair prefix in LDS then holds this sequence's pairs alone.
    int32_t spec_ids[kWindowPages / kWave];
    int spec_seq = -1;
    if (inl && p.whole_segments) {
        const int g = w / S, s = w - g * S;
        if (g >= p.Hkv) return;
        const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks;
#pragma unroll
        for (int c = 0; c < kWindowPages / kWave; ++c) {
            const int pg = c * kWave + lane;
            spec_ids[c] = pg < p.max_blocks ? bt[pg] : 0;
        }
        const int c = __builtin_amdgcn_readfirstlane(decode_pairs(
            p.qsl, p.seq_lens, p.kv_start, s, p.wmax, p.total_q, p.max_seqlen_k, p.max_blocks));
        if (c == 0) return;
        for (int i = lane; i <= S; i += kWave) lds_pref[i] = i <= s ? 0 : c;
        wave_lds_fence();
        u0 = (int64_t)g * c;
        u1 = u0 + c;
        spec_seq = s;
    } else if (inl) {
        // page pairs of every sequence and their exclusive prefix, in LDS
        const int per = (S + kWave - 1) / kWave;
        const int s_lo = min(S, lane * per), s_hi = min(S, s_lo + per);
        int sum = 0;
        for (int s = s_lo; s < s_hi; ++s) {
            const int c = decode_pairs(p.qsl, p.seq_lens, p.kv_start, s, p.wmax, p.total_q,
                                       p.max_seqlen_k, p.max_blocks);
            lds_pref[s] = c;
            sum += c;
        }
        int incl = sum;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int v = __shfl_up(incl, off);
            if (lane >= off) incl += v;
        }
        int run = incl - sum;
        for (int s = s_lo; s < s_hi; ++s) {
            const int c = lds_pref[s];
            lds_pref[s] = run;
            run += c;
        }
        if (lane == kWave - 1) lds_pref[S] = incl;
        wave_lds_fence();
        if (w == 0)
            for (int s = lane; s <= S; s += kWave) p.pair_prefix[s] = lds_pref[s];
        const int64_t U = (int64_t)p.Hkv * __builtin_amdgcn_readfirstlane(lds_pref[S]);
        u0 = wave_start(w, U);
        u1 = wave_start(w + 1, U);
        if (u0 >= u1) return;
    } else {
        pb = p.portion_begin[w];
        pe = p.portion_begin[w + 1];
        if (pb >= pe) return;
    }
    auto pref = [&](int s) { return __builtin_amdgcn_readfirstlane(lds_pref[s]); };
    // inline mode: the walk over the segments that meet [u0, u1) -- sequence
    // ws, kv head wg, ws's pairs wc, pieces emitted so far
    int ws = 0, wg = 0, wcount = 0;
    int64_t wc = 0;
    bool wdone = !inl;
    if (inl) {
        wg = (int)(u0 / pref(S));
        const int64_t r0 = u0 - (int64_t)wg * pref(S);
        int lo = 0, hi = S - 1;  // largest s with P[s] <= r0 (then P[s+1] > P[s])
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pref(mid) <= r0) lo = mid; else hi = mid - 1;
        }
        ws = lo;
        wc = pref(ws + 1) - pref(ws);
    }

    const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
    const uint8_t* vpool = static_cast<const uint8_t*>(p.v_pool);
    const int64_t page_stride = (int64_t)p.Hkv * kPage * Gm::RB;  // bytes per physical page
    // This lane's column is query token col / G, head col % G of the kv head's
    // group.  The quotient is recomputed where it is needed (a multiply by
    // ceil(2^16 / G) and a shift, exact for col < 16) rather than held in a
    // register across the streaming loop; the empty asm keeps the compiler from
    // hoisting it there.
    auto col_tok = [&]() {
        int m = p.gmagic;
        asm volatile("" : "+s"(m));
        return (col * m) >> 16;
    };

    if (spec_seq >= 0) {
#pragma unroll
        for (int c = 0; c < kWindowPages / kWave; ++c)
            lds_bid[c * kWave + lane] =
                (spec_ids[c] >= 0 && spec_ids[c] < p.num_blocks) ? spec_ids[c] : 0;
        wave_lds_fence();
    }

    for (int b0 = pb;;) {
        // ---- this batch's segment pieces (up to 64) into lds_port
        int n = 0, npairs = 0;
        wave_lds_fence();  // the previous batch is done with lds_port
        if (!inl) {
            if (b0 >= pe) break;
            n = min(kWave, pe - b0);
            if (lane < n) {
                const Portion q = p.portions[b0 + lane];
                lds_port[lane] = q;
                npairs = q.pi1 - q.pi0;
            }
            b0 += n;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) npairs += __shfl_xor(npairs, off);
        } else {
            if (wdone) break;
            while (n < kWave && !wdone) {
                const int64_t seg0 = segment_start(wg, pref(ws), pref(S));
                const int64_t seg1 = seg0 + wc;
                Portion q;
                q.s = ws;
                q.g = wg;
                q.pi0 = (int32_t)(max(u0, seg0) - seg0);
                q.pi1 = (int32_t)(min(u1, seg1) - seg0);
                q.slot = (seg0 >= u0 && seg1 <= u1) ? -1 : w * 2 + (wcount == 0 ? 0 : 1);
                q.q0 = p.qsl[ws];
                q.nq = p.qsl[ws + 1] - q.q0;
                const SeqRange r = seq_range(p.seq_lens, p.kv_start, ws, p.max_seqlen_k, p.max_blocks);
                q.kv_lo = r.a;
                q.kv_hi = r.L;
                if (lane == 0) lds_port[n] = q;
                npairs += q.pi1 - q.pi0;
                ++n;
                ++wcount;
                if (seg1 >= u1) {
                    wdone = true;
                } else {
                    do { ++ws; } while (ws < S && pref(ws + 1) == pref(ws));
                    if (ws == S) {
                        ++wg;
                        ws = 0;
                        while (pref(ws + 1) == pref(ws)) ++ws;
                    }
                    wc = pref(ws + 1) - pref(ws);
                }
            }
        }
        wave_lds_fence();
        const int K = npairs;
        // a field of piece idx (uniform), read back from LDS into a scalar register
#define PKV_FIELD(name, idx) __builtin_amdgcn_readfirstlane(lds_port[idx].name)

        // ---- issue cursor (runs two pairs ahead of the process cursor)
        int ip = 0, ipi = PKV_FIELD(pi0, 0), iend = PKV_FIELD(pi1, 0);
        int is = PKV_FIELD(s, 0), ig = PKV_FIELD(g, 0);
        int ifirst = PKV_FIELD(kv_lo, 0) / kPage;
        int iendpg = (PKV_FIELD(kv_hi, 0) + kPage - 1) / kPage;
        // the block-id window in LDS: pages [wstart, wstart + kWindowPages)
        // of sequence wseq's row (the speculative window of a whole segment)
        int wstart = spec_seq >= 0 ? 0 : -1, wseq = spec_seq;
        bool idone = false;

        auto issue = [&](PairRegs<T, D>& R) {
            const int pa = ifirst + 2 * ipi;
            const int pb2 = (pa + 1 < iendpg) ? pa + 1 : pa;
            if (wseq != is || pa < wstart || pb2 >= wstart + kWindowPages) {
                // stage the next window of this sequence's block-table row
                const int32_t* bt = p.block_tables + (int64_t)is * p.max_blocks;
                int32_t ids[kWindowPages / kWave];
#pragma unroll
                for (int c = 0; c < kWindowPages / kWave; ++c) {
                    const int pg = pa + c * kWave + lane;
                    ids[c] = pg < iendpg ? bt[pg] : 0;
                }
                wave_lds_fence();
#pragma unroll
                for (int c = 0; c < kWindowPages / kWave; ++c)
                    lds_bid[c * kWave + lane] =
                        (ids[c] >= 0 && ids[c] < p.num_blocks) ? ids[c] : 0;
                wave_lds_fence();
                wstart = pa;
                wseq = is;
            }
            const int64_t head_off = (int64_t)ig * kPage * Gm::RB;
            // A pair issued past the cursor's end (never consumed) and the
            // second page of a pair that has one page in range use empty
            // resources: the loads return zeros without touching memory.
            {
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int pg = x ? pb2 : pa;
                    const int64_t blk = __builtin_amdgcn_readfirstlane(lds_bid[pg - wstart]);
                    const int bytes = (idone || (x && pb2 == pa)) ? 0 : kPage * Gm::RB;
                    const auto kr = buffer_rsrc(kpool + blk * page_stride + head_off, bytes);
                    const auto vr = buffer_rsrc(vpool + blk * page_stride + head_off, bytes);
#pragma unroll
                    for (int i = 0; i < Gm::KCH; ++i)
                        R.k[x][i] = buffer_ld16<true>(kr, col * Gm::RB + i * 64 + grp * 16);
#pragma unroll
                    for (int c = 0; c < Gm::VCH; ++c)
                        R.v[x][c] = buffer_ld16<true>(vr, (c * kWave + lane) * 16);
                }
            }
            // advance; past the end the last pair is issued again (zeros, unused)
            if (!idone && ++ipi == iend) {
                if (ip + 1 < n) {
                    ++ip;
                    ipi = PKV_FIELD(pi0, ip);
                    iend = PKV_FIELD(pi1, ip);
                    is = PKV_FIELD(s, ip);
                    ig = PKV_FIELD(g, ip);
                    ifirst = PKV_FIELD(kv_lo, ip) / kPage;
                    iendpg = (PKV_FIELD(kv_hi, ip) + kPage - 1) / kPage;
                } else {
                    idone = true;
                    --ipi;
                }
            }
        };

        // ---- process cursor state: the segment piece being accumulated
        int pp = -1, ppi = 0, pend = 0;
        int ps = 0, pg_ = 0, pslot = 0, pq0 = 0, plo = 0, phi = 0, pfirst = 0;
        int plast = 0;   // last key the window's first token sees: seq_len - nq
        int pnq = 1;
        int pinner = 0;  // pairs [0, pinner) of the segment end at or before plast
        u32x4 qop[Gm::KCH];
        f32x4 acc[Gm::NT];
        float m_run = -INFINITY, l_run = 0.f;

        auto begin_piece = [&](int idx) {
            pp = idx;
            ppi = PKV_FIELD(pi0, idx);
            pend = PKV_FIELD(pi1, idx);
            ps = PKV_FIELD(s, idx);
            pg_ = PKV_FIELD(g, idx);
            pslot = PKV_FIELD(slot, idx);
            pq0 = PKV_FIELD(q0, idx);
            plo = PKV_FIELD(kv_lo, idx);
            phi = PKV_FIELD(kv_hi, idx);
            pnq = PKV_FIELD(nq, idx);
            plast = phi - pnq;
            pfirst = plo / kPage;
            pinner = max(0, (plast + 1 - pfirst * kPage) / (2 * kPage));
            const int ctok = col_tok();
            const bool hvalid = ctok < pnq;
            const uint8_t* qrow = static_cast<const uint8_t*>(p.q) +
                                  (hvalid ? ((int64_t)(pq0 + ctok) * p.Hq + pg_ * p.G + col - ctok * p.G) : 0) *
                                      Gm::RB;
#pragma unroll
            for (int i = 0; i < Gm::KCH; ++i) {
                u32x4 v = ld16(qrow + i * 64 + grp * 16);
                qop[i] = hvalid ? v : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int t = 0; t < Gm::NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_run = -INFINITY;
            l_run = 0.f;
            if (PS && ppi == 0) {
                // the segment's first piece starts from the prefix's state
                // (its chunks already folded into the first chunk's row)
                const int4 cd = p.prefix_states[ps];
                if (cd.x >= 0 && hvalid) {
                    const int h = pg_ * p.G + col - ctok * p.G;
                    const int64_t r = (cd.x < p.state_rows) ? cd.x : 0;
                    const float* sr = p.state + (r * p.Hq + h) * kStateStride<D>;
#pragma unroll
                    for (int t = 0; t < Gm::NT; ++t)
                        acc[t] = *reinterpret_cast<const f32x4*>(sr + t * 16 + grp * 4);
                    m_run = sr[D];
                    l_run = grp == 0 ? sr[D + 1] : 0.f;  // summed over the column's lanes at the end
                }
            }
        };

        auto finish_piece = [&]() {
            const float l_tot = col_sum(l_run);
            const int ctok = col_tok();
            if (ctok >= pnq) return;
            if (pslot < 0) {
                const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
                uint8_t* orow = static_cast<uint8_t*>(p.out) +
                                ((int64_t)(pq0 + ctok) * p.Hq + pg_ * p.G + col - ctok * p.G) * Gm::RB;
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
                const int64_t slot = (int64_t)pslot * p.ncol + col;
                float* o = p.ws_o + slot * D;
#pragma unroll
                for (int t = 0; t < Gm::NT; ++t)
                    *reinterpret_cast<f32x4*>(o + t * 16 + grp * 4) = acc[t];
                if (grp == 0) {
                    p.ws_ml[slot * 2] = m_run;
                    p.ws_ml[slot * 2 + 1] = l_tot;
                }
            }
        };

        // One pair of pages.  `edge` pairs (partly outside [kv_lo, kv_hi), or
        // reaching past the first window token's position) mask keys and zero
        // the V entries of keys outside [kv_lo, kv_hi); interior pairs skip all
        // masking.  The running max is raised lazily: only when a tile's max
        // exceeds it by more than 8 (log2 units), so probabilities stay below
        // 2^8 and the accumulator rescale is rare.
        auto process = [&](auto edge_tag, int pa, const PairRegs<T, D>& R) {
            constexpr bool EDGE = decltype(edge_tag)::value;
            const int kv_lo = plo, kv_hi = phi;
            const int cap = plast + (EDGE ? col_tok() : 0);  // last key this column's token sees
            // stage V (row-major, padded rows) for the transposed reads below
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int c = 0; c < Gm::VCH; ++c) {
                    const int ci = c * kWave + lane;
                    const int row = ci / Gm::CPR, cc = ci % Gm::CPR;
                    st16(lds_v + x * Gm::PAGE_LDS + row * Gm::RS + cc * 16, R.v[x][c]);
                }
            wave_lds_fence();

            // logits: lane holds keys 4*grp+{0..3} of each page for column col
            f32x4 sx[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (kBF) {
#pragma unroll
                    for (int i = 0; i < Gm::KCH; ++i) sacc = mfma_bf16(R.k[x][i], qop[i], sacc);
                } else {
#pragma unroll
                    for (int i = 0; i < Gm::KCH; ++i)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            sacc = mfma_f32(__uint_as_float(R.k[x][i][t]),
                                            __uint_as_float(qop[i][t]), sacc);
                }
                sx[x] = sacc;
            }
            // key (x, t) of this lane: (pa + x) * kPage + 4 * grp + t; stored keys
            // lie in [kv_lo, kv_hi) (V entries of the rest are zeroed below) and
            // this column's token sees the stored keys up to cap
            auto stored = [&](int x, int t) {
                const int key = (pa + x) * kPage + grp * 4 + t;
                return (unsigned)(key - kv_lo) < (unsigned)(kv_hi - kv_lo);
            };
            float sv[8];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int key = (pa + x) * kPage + grp * 4 + t;
                    const bool seen = !EDGE || (key >= kv_lo && key <= min(cap, kv_hi - 1));
                    sv[x * 4 + t] = seen ? sx[x][t] * p.scale_log2 : -INFINITY;
                }
            float mt = sv[0];
#pragma unroll
            for (int t = 1; t < 8; ++t) mt = fmaxf(mt, sv[t]);
            mt = col_max(mt);
            if (__any(mt > m_run + 8.f)) {
                const float m_new = fmaxf(m_run, mt);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = fast_exp2(m_run - m_use);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < Gm::NT; ++t) acc[t] *= alpha;
            }
            const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
            float pv[8];
            float psum = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                pv[t] = fast_exp2(sv[t] - m_use);
                psum += pv[t];
            }
            l_run += psum;

            // O^T += V^T P^T, V^T from the staged pages
            if constexpr (kBF) {
                u32x4 pbv = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]),
                             pack_bf16(pv[4], pv[5]), pack_bf16(pv[6], pv[7])};
                // transposing reads: the 16 lanes of group grp point at keys
                // 4 grp .. 4 grp + 3 of a page, 4 lanes per key and 8 bytes
                // each over tile t's 16 columns, and lane col receives column
                // 16 t + col of those 4 keys -- the keys its P^T entries hold
                const uint8_t* vb = lds_v + (4 * grp + (col >> 2)) * Gm::RS + (col & 3) * 8;
                uint32_t keep[4];
                if constexpr (EDGE) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int x = q >> 1, t = (q & 1) * 2;
                        keep[q] = (stored(x, t) ? 0x0000ffffu : 0u) |
                                  (stored(x, t + 1) ? 0xffff0000u : 0u);
                    }
                }
#pragma unroll
                for (int t = 0; t < Gm::NT; ++t) {
                    const uint2 lo = lds_read_tr16(vb + t * 32);
                    const uint2 hi = lds_read_tr16(vb + Gm::PAGE_LDS + t * 32);
                    u32x4 a = {lo.x, lo.y, hi.x, hi.y};
                    if constexpr (EDGE) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) a[q] &= keep[q];
                    }
                    acc[t] = mfma_bf16(a, pbv, acc[t]);
                }
            } else {
                const float* lf = reinterpret_cast<const float*>(lds_v);
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int key = grp * 4 + u;
#pragma unroll
                        for (int t = 0; t < Gm::NT; ++t) {
                            float v = lf[(x * Gm::PAGE_LDS + key * Gm::RS) / 4 + t * 16 + col];
                            if constexpr (EDGE) v = stored(x, u) ? v : 0.f;
                            acc[t] = mfma_f32(v, pv[x * 4 + u], acc[t]);
                        }
                    }
            }
            wave_lds_fence();
        };

        auto consume = [&](const PairRegs<T, D>& R) {
            if (pp < 0 || ppi == pend) {
                if (pp >= 0) finish_piece();
                begin_piece(pp + 1);
            }
            const int pa = pfirst + 2 * ppi;
            if ((ppi == 0 && plo != pfirst * kPage) || ppi >= pinner)
                process(std::true_type{}, pa, R);
            else
                process(std::false_type{}, pa, R);
            ++ppi;
        };

        if (K > 0) {
            PairRegs<T, D> A, B;
            // With one wave per segment the segment's queries load before its
            // pages: loads complete in order, so queries loaded after the
            // first two pairs hold the first products until both pairs have
            // arrived, a pair's latency of a short segment.  Spread over the
            // waves, where the first pages matter more than the first
            // products, the pages go first.
            if (p.whole_segments) begin_piece(0);
            issue(A);
            issue(B);
            for (int k = 0; k < K; k += 2) {
                consume(A);
                issue(A);
                if (k + 1 < K) consume(B);
                issue(B);
            }
            finish_piece();
        }
    }
    asm volatile("" ::"v"(bt_touch));
}

#undef PKV_FIELD

template <typename T, int D, bool PS>
__global__ void __launch_bounds__(64, __is_same(T, float) ? 1 : 2) decode_kernel(DecodeParams p) {
    __shared__ DecodeLds<T, D> lds;
    decode_wave<T, D, PS>(p, p.whole_segments ? (int)blockIdx.x : decode_wave_id(), lds);
}

// One wavefront per (sequence, query head) whose segment was cut by a wave
// boundary, for each of the sequence's query tokens:
// out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j over its pieces,
// rounded to the output type.  Lane j takes the j-th decode wave of
// the segment (waves whose unit range is empty hold nothing: they lie between
// the segment's waves when there are fewer units than waves); maxima and sums
// combine across lanes, then every lane sums its output elements over the
// pieces that exist, eight loads in flight at a time.
template <typename T, int D>
__global__ void __launch_bounds__(64) merge_kernel(MergeParams p) {
    constexpr bool kBF = !__is_same(T, float);
    constexpr int PER = D / kWave;  // output elements per lane (1 or 2)
    int h, s;
    if (p.Hkv % kXcds == 0) {
        // Workgroup b runs on XCD b % 8: give it a (sequence, head) whose kv
        // head that XCD's decode waves streamed (with the kv heads a multiple
        // of the XCDs each XCD takes whole heads), so that the partials it
        // reads can still sit in that XCD's L2 (back-to-back steps: ~1 us).
        const int x = (int)(blockIdx.x % kXcds), k = (int)(blockIdx.x / kXcds);
        const int per = p.Hq / kXcds;
        s = k / per;
        h = x * per + k % per;
    } else {
        h = blockIdx.x % p.Hq;
        s = blockIdx.x / p.Hq;
    }
    if (s >= p.num_seqs) return;
    const int64_t c = p.pair_prefix[s + 1] - p.pair_prefix[s];
    if (c <= 0) return;
    const int64_t U = (int64_t)p.Hkv * p.pair_prefix[p.num_seqs];
    const int g = h / p.G, head = h - (h / p.G) * p.G;
    const int64_t a = segment_start(g, p.pair_prefix[s], p.pair_prefix[p.num_seqs]);
    const int64_t wa = wave_of(a, U), wb = wave_of(a + c - 1, U);
    if (wa == wb) return;  // the wave that holds the whole segment wrote it
    const int lane = threadIdx.x;
    const int q0 = p.qsl[s];
    const int nq = p.qsl[s + 1] - q0;
    auto holds = [&](int64_t w) { return w <= wb && wave_start(w, U) < wave_start(w + 1, U); };
    // first-piece slot of wave w, or its second piece when w's range starts before a
    auto slot_row = [&](int64_t w) -> int32_t {
        const int which = (w == wa && wave_start(wa, U) != a) ? 1 : 0;
        return (int32_t)((w * 2 + which) * p.ncol);
    };

    for (int tok = 0; tok < nq; ++tok) {
        const int column = tok * p.G + head;
        float M = -INFINITY;
        for (int64_t w0 = wa; w0 <= wb; w0 += kWave) {
            const int64_t w = w0 + lane;
            if (holds(w)) M = fmaxf(M, p.ws_ml[(int64_t)(slot_row(w) + column) * 2]);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        const float Mu = (M == -INFINITY) ? 0.f : M;

        float num[PER], den = 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) num[e] = 0.f;
        for (int64_t w0 = wa; w0 <= wb; w0 += kWave) {
            const int64_t w = w0 + lane;
            const bool mine = holds(w);
            const int32_t sl = (mine ? slot_row(w) : slot_row(wa)) + column;
            const float wt = mine ? fast_exp2(p.ws_ml[(int64_t)sl * 2] - Mu) : 0.f;
            if (mine) den += wt * p.ws_ml[(int64_t)sl * 2 + 1];
            // the lanes whose wave holds a piece, lowest first (when a step has
            // fewer units than waves, most waves of a segment's span are empty)
            uint64_t rem = __ballot(mine);
            const int cnt = __popcll(rem);
            for (int j0 = 0; j0 < cnt; j0 += 8) {
                float o[8][PER];
                bool use[8];
                float wj[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    use[k] = rem != 0;
                    const int j = use[k] ? __ffsll((unsigned long long)rem) - 1 : 0;
                    rem &= rem - 1;
                    const int32_t slj = __builtin_amdgcn_readlane(sl, j);
                    wj[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), j));
                    const float* src = p.ws_o + (int64_t)slj * D + lane * PER;
#pragma unroll
                    for (int e = 0; e < PER; ++e) o[k][e] = src[e];
                }
#pragma unroll
                for (int k = 0; k < 8; ++k)
#pragma unroll
                    for (int e = 0; e < PER; ++e) num[e] += use[k] ? wj[k] * o[k][e] : 0.f;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
        const float inv = den > 0.f ? 1.f / den : 0.f;
        uint8_t* orow = static_cast<uint8_t*>(p.out) +
                        ((int64_t)(q0 + tok) * p.Hq + h) * (int64_t)D * Elem<T>::kBytes;
        if constexpr (kBF) {
            if constexpr (PER == 2) {
                reinterpret_cast<uint32_t*>(orow)[lane] = pack_bf16(num[0] * inv, num[1] * inv);
            } else {
                reinterpret_cast<uint16_t*>(orow)[lane] =
                    (uint16_t)(pack_bf16(num[0] * inv, 0.f) & 0xffffu);
            }
        } else {
#pragma unroll
            for (int e = 0; e < PER; ++e)
                reinterpret_cast<float*>(orow)[lane * PER + e] = num[e] * inv;
        }
    }
}

}  // namespace pkv
