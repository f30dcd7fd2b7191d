// Shared-prefix ("cascade") steps: groups of decode sequences whose first
// keys sit in common physical pages read those pages once per group and kv
// head, instead of once per sequence.
//
// The pages name the case: requests that share a prompt prefix keep it in
// shared pages (vllm-metal v0.4.0 release post, "Prefix caching on hybrid
// models"; the vllm-mlx paper summary, results: prefix caching measured on
// 512-token shared prefixes).  Attention over the union of two key sets is the
// log-sum-exp combination of the attention over each, so a step splits into
//   1. the prefix pass: for every group, chunk of its prefix and kv head, one
//      matrix-core tile computes the softmax states (max, sum, unnormalised
//      output) of all the group's query rows over that chunk -- the
//      chunked-prefill kernel run on a virtual step whose sequences are the
//      chunks and whose tokens are the group's decode tokens;
//   2. the combination of each member's chunk states into one (below);
//   3. the decode pass over each sequence's own keys only (kv_start = prefix
//      length), whose first piece per segment starts from the prefix state;
//      the merge of cut segments is unchanged.
// The setup kernel builds the virtual step of (1) and the per-sequence inputs
// of (2) and (3) on the device, from the caller's group arrays.
#pragma once

#include "pkv_device.hpp"
#include "decode.hpp"

namespace pkv {

constexpr int kCascadeThreads = 1024;
constexpr int kCascadeMaxSeqs = 16384;   // sequences a step may hold
constexpr int kCascadeMaxGroups = 1024;  // groups per step
// the entry point admits up to kMaxDecodeSeqs sequences; the setup kernel
// must give every one of them its prefix inputs
static_assert(kCascadeMaxSeqs >= kMaxDecodeSeqs, "setup kernel covers fewer sequences than a step");
static_assert(kCascadeMaxSeqs % kCascadeThreads == 0, "sequences split evenly over threads");

struct CascadeParams {
    const int32_t* prefix_group;  // [num_seqs]: group of sequence s, or -1
    const int32_t* prefix_len;    // [num_groups]: shared keys (a multiple of 16)
    const int32_t* qsl;           // [num_seqs + 1]
    const int32_t* seq_lens;      // [num_seqs]
    int num_seqs;
    int num_groups;
    int max_members;  // members per group kept (any others run as plain sequences)
    int max_chunks;   // chunks per group
    int chunk;        // keys per chunk (a multiple of 32)
    int64_t total_q;
    // outputs, in the workspace
    int32_t* kv_eff;        // [num_seqs] keys each sequence's decode pass skips
    int4* prefix_states;    // [num_seqs] (first state row, row stride, chunks)
    int32_t* v_qsl;         // [V + 1] virtual step, V = num_groups * max_chunks
    int32_t* v_lens;        // [V] chunk end (keys)
    int32_t* v_start;       // [V] chunk start (keys)
    int32_t* v_row;         // [V] block-table row holding the group's pages
    int32_t* v_qrows;       // [V * max_members] query row of each virtual token
};

// LDS the setup kernel needs for a step (dynamic: sized to the step's groups).
inline size_t cascade_setup_lds(int num_groups) {
    return sizeof(int32_t) * (5 * (size_t)num_groups + 1 + kPlanThreads);
}

// Sequences are spread over the threads (at most 16 each); a member takes a
// slot in its group with an LDS atomic.  Slot order is arbitrary: the prefix
// pass computes each query row independently of the other rows of its tile,
// so no output bit depends on it; when a group has more members than
// max_members, which of them run as plain sequences is unspecified.
__global__ void __launch_bounds__(kCascadeThreads) cascade_setup_kernel(CascadeParams p) {
    extern __shared__ int32_t smem[];
    const int t = threadIdx.x;
    const int S = min(p.num_seqs, kCascadeMaxSeqs);
    const int NG = min(p.num_groups, kCascadeMaxGroups);
    const int CH = p.max_chunks;
    int32_t* count = smem;              // [NG] members that asked for a slot
    int32_t* members = count + NG;      // [NG] members kept (capped)
    int32_t* rep = members + NG;        // [NG] lowest member: its block-table row
    int32_t* plen = rep + NG;           // [NG] prefix keys
    int32_t* base = plen + NG;          // [NG + 1] first virtual token of each group
    int32_t* tmp = base + NG + 1;       // [kPlanThreads] scan scratch

    for (int g = t; g < NG; g += kCascadeThreads) {
        int P = p.prefix_len[g];
        P = P < 0 ? 0 : min(P, CH * p.chunk) & ~(kPage - 1);
        plen[g] = P;
        count[g] = 0;
        rep[g] = 0x7fffffff;
    }
    __syncthreads();
    // a sequence joins its group only as a decode (one query token) with
    // keys past the prefix
    constexpr int PER = kCascadeMaxSeqs / kCascadeThreads;
    int my_g[PER], my_j[PER], my_q0[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int s = t + k * kCascadeThreads;
        my_g[k] = -1;
        my_j[k] = 0;
        my_q0[k] = 0;
        if (s >= S) continue;
        int g = p.prefix_group[s];
        const int q0 = p.qsl[s], nq = p.qsl[s + 1] - q0, L = p.seq_lens[s];
        if (g < 0 || g >= NG || nq != 1 || q0 < 0 || q0 >= p.total_q || plen[g] == 0 ||
            L <= plen[g])
            continue;
        my_g[k] = g;
        my_q0[k] = q0;
        my_j[k] = atomicAdd(&count[g], 1);
        atomicMin(&rep[g], s);
    }
    __syncthreads();
    for (int g = t; g < NG; g += kCascadeThreads) {
        members[g] = min(count[g], p.max_members);
        base[g] = members[g] * ((plen[g] + p.chunk - 1) / p.chunk);
        if (rep[g] == 0x7fffffff) rep[g] = 0;
    }
    __syncthreads();
    block_exclusive_scan(base, NG, tmp);
    // the virtual step: sequence v = g * CH + c is chunk c of group g's prefix
    for (int v = t; v < NG * CH; v += kCascadeThreads) {
        const int g = v / CH, c = v - (v / CH) * CH;
        const int P = plen[g];
        const int chunks = (P + p.chunk - 1) / p.chunk;
        const bool live = c < chunks && members[g] > 0;
        p.v_qsl[v] = base[g] + min(c, chunks) * members[g];
        p.v_start[v] = live ? c * p.chunk : 0;
        p.v_lens[v] = live ? min((c + 1) * p.chunk, P) : 0;
        p.v_row[v] = rep[g];
    }
    if (t == 0) p.v_qsl[NG * CH] = base[NG];
    // member j of group g is token j of every live chunk of the group
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int s = t + k * kCascadeThreads;
        if (s >= p.num_seqs) continue;
        const int g = my_g[k], j = my_j[k];
        if (g >= 0 && j < members[g]) {
            const int chunks = (plen[g] + p.chunk - 1) / p.chunk;
            for (int c = 0; c < chunks; ++c) p.v_qrows[base[g] + c * members[g] + j] = my_q0[k];
            p.prefix_states[s] = int4{base[g] + j, members[g], chunks, 0};
            p.kv_eff[s] = plen[g];
        } else {  // not a member, or past the group's cap: a plain sequence
            p.prefix_states[s] = int4{-1, 0, 0, 0};
            p.kv_eff[s] = 0;
        }
    }
}

// Folds the chunk states of every (member, query head) into one, written over
// the first chunk's state row: M = max_c m_c, l = sum_c 2^(m_c - M) l_c,
// o = sum_c 2^(m_c - M) o_c.  One wavefront per (sequence, query head); lane c
// reads chunk c's maximum, every lane then sums D / 64 output elements over
// the chunks with eight chunk rows in flight.
struct StateCombineParams {
    const int4* prefix_states;  // [num_seqs]
    float* state;               // [rows][Hq][kStateStride]
    int64_t state_rows;
    int num_seqs;
    int Hq;
};

template <int D>
__global__ void __launch_bounds__(64) state_combine_kernel(StateCombineParams p) {
    constexpr int SS = kStateStride<D>;
    constexpr int PER = D / kWave;
    const int h = blockIdx.x % p.Hq;
    const int s = blockIdx.x / p.Hq;
    if (s >= p.num_seqs) return;
    const int4 cd = p.prefix_states[s];
    if (cd.x < 0 || cd.z <= 1) return;
    const int lane = threadIdx.x;
    auto row = [&](int c) {
        int64_t r = (int64_t)cd.x + (int64_t)c * cd.y;
        r = (r >= 0 && r < p.state_rows) ? r : 0;
        return p.state + (r * p.Hq + h) * SS;
    };
    float M = -INFINITY;
    for (int c0 = 0; c0 < cd.z; c0 += kWave)
        if (c0 + lane < cd.z) M = fmaxf(M, row(c0 + lane)[D]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float l = 0.f, o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
    for (int c0 = 0; c0 < cd.z; c0 += 8) {
        float w[8], v[8][PER], lc[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = min(c0 + k, cd.z - 1);
            const float* sr = row(c);
            w[k] = c0 + k < cd.z ? fast_exp2(sr[D] - Mu) : 0.f;
            lc[k] = sr[D + 1];
#pragma unroll
            for (int e = 0; e < PER; ++e) v[k][e] = sr[lane * PER + e];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            l += w[k] * lc[k];
#pragma unroll
            for (int e = 0; e < PER; ++e) o[e] += w[k] * v[k][e];
        }
    }
    float* dst = row(0);
    __syncthreads();  // every lane has read row 0 before it is overwritten
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[lane * PER + e] = o[e];
    if (lane == 0) {
        dst[D] = M;
        dst[D + 1] = l;
    }
}

}  // namespace pkv
