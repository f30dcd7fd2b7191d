// Chunked-prefill attention for sequences with more query tokens in the step
// than the decode path takes (a chunk of a prompt).
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
// Work unit: one workgroup per (sequence, kv head, tile of query tokens).
// The G query heads of the kv head are folded into the tile's rows
// (row = token * G + head), so every staged K/V page serves all of them.
// Keys are the MFMA rows:  S^T = K q^T,  O^T += V^T P^T.  Four row blocks of
// 32 rows (two 16-column MFMA tiles) cover the tile's 128 rows.  For bfloat16
// each row block has two wavefronts on the same SIMD that take alternate KV
// stages (eight wavefronts per workgroup), so that one can issue while the
// other waits on a dependency; their partial results are combined through LDS
// at the end with the usual log-sum-exp rescaling.
//
// Staging: pairs of KV pages (32 keys; K and V of two pages, 16 KiB for bf16
// head_dim 128) go from HBM straight into a ring of kStages LDS buffers with
// global->LDS loads, issued several rounds ahead of the stages being consumed,
// one workgroup barrier per round.  Inside a buffer each 16-byte chunk of a
// row sits at chunk ^ f(row), with f chosen per page kind (K or V) so that
// the rows one read instruction touches fall in distinct banks.  V^T operands
// come from the transposing LDS read (ds_read_b64_tr_b16), which hands each
// lane 4 consecutive keys of one column.  A wavefront issues at most one
// instruction per 4-cycle turn of its SIMD, so the transfer bookkeeping is
// kept to a few scalar instructions per stage (pre-scaled page offsets in LDS,
// scalar-base loads).  The sequence that owns a tile is found from
// query_start_loc: up to kPrefillCompactSeqs sequences by a prefix sum of
// their tile counts that every wavefront computes (tiles numbered over the
// prefill sequences only, the last tile first), beyond that by a binary
// search over tile slots ("Replacing attention, reusing the rest": each
// threadgroup finds its request by binary search over cu_seqlens).
#pragma once

#include <type_traits>

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
    int min_q;         // sequences with fewer query tokens take the decode path
    int max_seqlen_k;
    int64_t total_q;
    int64_t num_blocks;
    float scale_log2;
    // Shared-prefix (state) pass; all null for a plain step.  With `state`
    // set, the step's sequences are chunks of shared prefixes: every token of
    // a sequence sees all of its keys [kv_start, seq_len) (no causal cap), its
    // query row is q_rows[token] (< q_limit), its block-table row is
    // seq_row[s] (< bt_rows), and each (token, head) writes its softmax state
    // -- unnormalised output [D], running max (log2 units), sum -- to
    // state[(token * Hq + head) * kStateStride] instead of an output row.
    const int32_t* q_rows;
    const int32_t* seq_row;
    float* state;
    int64_t q_limit;
    int bt_rows;
    int sp_tiles;  // state pass: tiles per sequence (grid = num_seqs x sp_tiles x Hkv)
};

constexpr int kPrefillCompactSeqs = 512;  // up to this many sequences in a step,
                                         // tiles are numbered over the prefill
                                         // sequences only
constexpr int kPrefillRowBlocks = 4;                 // 32-row blocks per workgroup
constexpr int kPrefillRows = 32 * kPrefillRowBlocks;

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes from global memory straight into LDS: lane l writes block + 16 * l
// (block is wave-uniform; M0 holds its LDS address).  Written as inline
// assembly so that the compiler does not treat later LDS reads of other ring
// slots as possibly aliasing the transfer and wait for every load in flight:
// the kernel orders these transfers itself, with explicit vmcnt waits and a
// workgroup barrier before a staged buffer is read.
__device__ __forceinline__ void load_to_lds16(const void* g, uint8_t* block) {
    // block is wave-uniform; made scalar explicitly, as M0 takes a scalar register
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)block);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(m0), "v"(g)
                 : "memory", "m0");
}

// The same with a wave-uniform 64-bit base in scalar registers and a 32-bit
// per-lane byte offset (the global address is base + off), and the LDS block
// given as an LDS byte address: no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void load_to_lds16(const uint8_t* base, uint32_t off, uint32_t lds_addr) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0), "v"(off), "s"(base)
                 : "memory", "m0");
}

// Raises (1) or lowers (0) this wavefront's issue priority, pinned in place.
// Around its matrix-core products a wavefront takes priority over the other
// wavefront of its SIMD, so the two drift apart and one's softmax overlaps the
// other's products.
__device__ __forceinline__ void mfma_priority(int hi) {
    __builtin_amdgcn_sched_barrier(0);
    if (hi) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier without the memory fence of __syncthreads(): a fence
// would make the compiler wait for every global->LDS load in flight, including
// the stages loaded ahead.  Visibility of a stage is ensured by the explicit
// vmcnt wait that precedes this barrier; the empty asm statements keep the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_keep_loads_in_flight() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // vmcnt in bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) left free
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wavefronts per 32-row block: two for bfloat16 (alternate stages), one for float32
template <typename T>
constexpr int kPrefillSplit = __is_same(T, float) ? 1 : 2;
template <typename T>
constexpr int kPrefillThreads = kPrefillRowBlocks * kPrefillSplit<T> * kWave;

template <typename T, int D>
struct PrefillGeom {
    static constexpr bool kBF = !__is_same(T, float);
    static constexpr int SPLIT = kPrefillSplit<T>;
    static constexpr int NW = kPrefillRowBlocks * SPLIT;   // wavefronts per workgroup
    static constexpr int kThreads = kPrefillThreads<T>;
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int RB = D * EB;                      // bytes per K/V row
    static constexpr int CPR = RB / 16;                    // 16-byte chunks per row
    static constexpr int PAGE = kPage * RB;                // bytes of one (page, head)
    static constexpr int STAGE = 4 * PAGE;                 // K a, K b, V a, V b
    static constexpr int BLOCKS = STAGE / 1024;            // 1 KiB load blocks per stage
    static constexpr int LPT = BLOCKS / NW;                // load instructions per thread
    static constexpr int ROWS_PER_BLOCK = 1024 / RB;
    // ring slots (a multiple of SPLIT; the ring stays within 128 KiB)
    static constexpr int kStages = (STAGE <= 16384) ? (kBF ? 8 : 4) : 2;
    static constexpr int NT = D / 16;
    static constexpr int KCH = RB / 64;
    // floats per lane handed from the second wavefront of a row block to the first
    static constexpr int XF = 2 * NT * 4 + 4;
    static_assert(LPT >= 1 && kStages % SPLIT == 0, "stage geometry");
    static_assert(SPLIT == 1 || kPrefillRowBlocks * kWave * XF * 4 <= kStages * STAGE,
                  "exchange area fits in the ring");
};

// Chunk position of row r's chunk c inside a staged LDS page.  K pages are
// read one 16-byte chunk of each of 16 rows per instruction (the MFMA A
// operand): XOR with the row spreads those over all banks.  V pages are read
// by the transposing read, 8 bytes of 4 consecutive rows per 16 lanes: XOR
// with twice the row keeps those 4 rows apart.  Both choices measured free of
// bank conflicts on gfx950; the other way round each costs half the rate.
template <int CPR>
__device__ __forceinline__ int swz_k(int r, int c) {
    return c ^ (r & (CPR - 1));
}
template <int CPR>
__device__ __forceinline__ int swz_v(int r, int c) {
    return c ^ ((((r & 7) << 1) | ((r >> 3) & 1)) & (CPR - 1));
}

// Waits until at most `later` stages of this thread's global->LDS loads (LPT
// instructions each) are still in flight; later <= MAXL.
template <int LPT, int MAXL>
__device__ __forceinline__ void wait_stages(int later) {
    if constexpr (MAXL == 0) {
        wait_vmcnt<0>();
    } else {
        if (later >= MAXL) wait_vmcnt<MAXL * LPT>();
        else wait_stages<LPT, MAXL - 1>(later);
    }
}

template <int K, int U, typename F>
__device__ __forceinline__ void unroll_rounds(F&& f) {
    if constexpr (K < U) {
        f(std::integral_constant<int, K>{});
        unroll_rounds<K + 1, U>(f);
    }
}

// Block-table entries a workgroup stages in LDS, as pool offsets (contexts
// up to 64K keys, pools whose offsets / 256 fit 32 bits); longer contexts and
// larger pools use the LONG variant, which reads the block ids through the
// scalar data cache instead.
constexpr int kPrefillIdTable = 4096;

// LDS of one prefill workgroup: the staging ring, and (!LONG) the byte
// offset / 256 of each staged (page, kv head) inside a pool, page-major:
// [page of the stage (0, 1)][stage], each row padded so that reads a round
// past the last stage stay inside it.
constexpr int kPrefillIdRow = kPrefillIdTable / 2 + 16;
template <typename T, int D, bool LONG>
struct PrefillLds {
    __attribute__((aligned(1024))) uint8_t ring[PrefillGeom<T, D>::kStages * PrefillGeom<T, D>::STAGE];
    __attribute__((aligned(8))) uint32_t bid[LONG ? 2 : 2 * kPrefillIdRow];
};

// The tile of workgroup number `block` (tile * Hkv + kv head), computed by the
// whole workgroup with the LDS `L`.  Runs as a workgroup of prefill_kernel,
// or as the second phase of a workgroup of the single-launch step kernel.
template <typename T, int D, bool LONG>
__device__ __forceinline__ void prefill_tile(const PrefillParams& p, const int block,
                                             PrefillLds<T, D, LONG>& L) {
    using Gm = PrefillGeom<T, D>;
    constexpr bool kBF = Gm::kBF;
    constexpr int NS = Gm::kStages;
    constexpr int SPLIT = Gm::SPLIT;
    constexpr int NW = Gm::NW;
    uint8_t* const lds = L.ring;
    constexpr int kIdRow = kPrefillIdRow;
    uint32_t* const lds_bid = L.bid;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int rblk = wave % kPrefillRowBlocks;  // 32-row block of this wavefront
    const int half = wave / kPrefillRowBlocks;  // stages st with st % SPLIT == half
    // Workgroup id = tile * Hkv + kv head: workgroups are handed to the eight
    // XCDs round-robin, so with Hkv a multiple of 8 every query tile of one kv
    // head runs on one XCD and re-reads that head's K/V pages from its L2.
    const int g = (int)((unsigned)block % (unsigned)p.Hkv);
    const int bid = (int)((unsigned)block / (unsigned)p.Hkv);
    const int BQ = p.tile_tokens;

    // ---- which sequence owns this tile, and which of its tiles it is
    const bool SP = p.state != nullptr;  // shared-prefix state pass
    int s = 0, qt = 0;
    if (SP) {
        // the state pass: sp_tiles tiles per sequence, in order
        s = bid / p.sp_tiles;
        if (s >= p.num_seqs) return;
        qt = bid - s * p.sp_tiles;
    } else if (p.num_seqs <= kPrefillCompactSeqs) {
        // Tiles numbered over the prefill sequences only (decode sequences
        // take none), from one read of the query offsets by every wavefront
        // (the result is uniform): the workgroups with a tile are then the
        // first ones, which start first, and none waits behind a workgroup
        // that had nothing to do.  The last tile comes first -- within a
        // chunk the later tiles see more keys -- so that when there are more
        // tiles than compute units the longest start first.
        const int S = p.num_seqs;
        const int per = (S + kWave - 1) / kWave;
        const int s_lo = min(S, lane * per), s_hi = min(S, s_lo + per);
        auto tiles_of = [&](int t) {
            const int a = p.qsl[t];
            int m = p.qsl[t + 1] - a;
            if (a < 0 || a >= p.total_q || m < max(2, p.min_q)) return 0;
            if (m > p.total_q - a) m = (int)(p.total_q - a);
            return (m + BQ - 1) / BQ;
        };
        int own = 0;
        for (int t = s_lo; t < s_hi; ++t) own += tiles_of(t);
        int incl = own;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int v = __shfl_up(incl, off);
            if (lane >= off) incl += v;
        }
        const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
        const int c = total - 1 - bid;
        if (c < 0) return;  // uniform: no tile left for this workgroup
        const int excl = incl - own;
        const bool holder = c >= excl && c < incl;
        int hs = 0, hq = 0;
        if (holder) {
            int run = excl;
            for (int t = s_lo; t < s_hi; ++t) {
                const int k = tiles_of(t);
                if (c < run + k) {
                    hs = t;
                    hq = c - run;
                    break;
                }
                run += k;
            }
        }
        const int src = __ffsll((unsigned long long)__ballot(holder)) - 1;
        s = __builtin_amdgcn_readlane(hs, src);
        qt = __builtin_amdgcn_readlane(hq, src);
    } else {
        // beyond that many sequences: tile slot bid of the sequence with the
        // largest s such that qsl[s] / BQ + s <= bid (slots of decode
        // sequences and of the rounding stay empty)
        int lo = 0, hi = p.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.qsl[mid] / BQ + mid <= bid) lo = mid; else hi = mid - 1;
        }
        s = lo;
        qt = bid - (p.qsl[s] / BQ + s);
    }
    int q0 = p.qsl[s];
    int n = p.qsl[s + 1] - q0;
    if (q0 < 0 || q0 >= p.total_q || n < (SP ? 1 : max(2, p.min_q))) return;
    if (n > p.total_q - q0) n = (int)(p.total_q - q0);
    const int tok0 = qt * BQ;
    if (qt < 0 || tok0 >= n) return;
    const int ntok = min(BQ, n - tok0);

    const SeqRange r = seq_range(p.seq_lens, p.kv_start, s, p.max_seqlen_k, p.max_blocks);
    // position of the tile's first token and of its last (the state pass: every
    // token sits past the last key)
    const int pos_min = SP ? r.L - 1 : r.L - n + tok0;
    const int pos_max = SP ? r.L - 1 : pos_min + ntok - 1;
    if (pos_max < r.a ||
        (!LONG && 2 * ((pos_max / kPage - r.first_page + 2) / 2) > kPrefillIdTable)) {
        // every row sees no key (only with metadata outside the contract): write
        // zeros, or the empty state
        for (int rr = tid; rr < ntok * p.G; rr += blockDim.x) {
            const int tok = rr / p.G, hh = rr % p.G;
            if (SP) {
                float* sr = p.state + ((int64_t)(q0 + tok0 + tok) * p.Hq + g * p.G + hh) * kStateStride<D>;
                for (int d = 0; d < D; ++d) sr[d] = 0.f;
                sr[D] = -INFINITY;
                sr[D + 1] = 0.f;
                continue;
            }
            uint8_t* orow = static_cast<uint8_t*>(p.out) +
                            ((int64_t)(q0 + tok0 + tok) * p.Hq + g * p.G + hh) * Gm::RB;
            for (int c = 0; c < Gm::CPR; ++c) st16(orow + c * 16, u32x4{0, 0, 0, 0});
        }
        return;
    }
    const int first_page = r.first_page;
    const int last_page = pos_max / kPage;
    const int npages = last_page - first_page + 1;
    const int nstage = (npages + 1) / 2;

    // ---- rows of this wavefront: two 16-column tiles; query operands first, so
    // that their loads complete before any staged K/V load
    int pos[2];
    bool rvalid[2];
    int64_t orow_idx[2];
    u32x4 qop[2][Gm::KCH];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int row = rblk * 32 + nt * 16 + col;
        const int tok = row / p.G, hh = row - (row / p.G) * p.G;
        rvalid[nt] = tok < ntok;
        pos[nt] = rvalid[nt] ? (SP ? pos_max : pos_min + tok) : -1;
        orow_idx[nt] = (int64_t)(q0 + tok0 + (rvalid[nt] ? tok : 0)) * p.Hq + g * p.G + hh;
        int64_t qidx = orow_idx[nt];
        if (SP) {  // the state pass reads the query row of the token's sequence
            int64_t qt = p.q_rows[q0 + tok0 + (rvalid[nt] ? tok : 0)];
            qt = (qt >= 0 && qt < p.q_limit) ? qt : 0;
            qidx = qt * p.Hq + g * p.G + hh;
        }
        const uint8_t* qrow = static_cast<const uint8_t*>(p.q) + qidx * Gm::RB;
#pragma unroll
        for (int i = 0; i < Gm::KCH; ++i) {
            u32x4 v = ld16(qrow + i * 64 + grp * 16);
            qop[nt][i] = rvalid[nt] ? v : u32x4{0, 0, 0, 0};
        }
    }

    const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
    const uint8_t* vpool = static_cast<const uint8_t*>(p.v_pool);
    const int64_t page_stride = (int64_t)p.Hkv * Gm::PAGE;
    const int64_t head_off = (int64_t)g * Gm::PAGE;

    // Stage st: wavefront w loads blocks w, w + NW, ...; block b covers rows
    // (b % (PAGE/1KiB)) * ROWS_PER_BLOCK.. of buffer b / (PAGE/1KiB).  The
    // lane's byte offset inside the (page, head) is fixed; per stage only the
    // two page bases change.
    constexpr int BPP = Gm::PAGE / 1024;  // blocks per page
    int src_off[Gm::LPT];
#pragma unroll
    for (int c = 0; c < Gm::LPT; ++c) {
        const int blk = c * NW + wave;
        const int row = (blk % BPP) * Gm::ROWS_PER_BLOCK + lane / Gm::CPR;
        const bool kbuf = blk / BPP < 2;   // buffers 0, 1 hold K, 2, 3 hold V
        src_off[c] = row * Gm::RB + (kbuf ? swz_k<Gm::CPR>(row, lane % Gm::CPR)
                                          : swz_v<Gm::CPR>(row, lane % Gm::CPR)) * 16;
    }
    // What stage st's transfers need from the block table (an odd page
    // count repeats the last page; ids outside the pool read page 0), fetched
    // a round ahead of their use.  Up to 64K keys the workgroup stages, once,
    // the byte offset / 256 of every (page, kv head) it reads in LDS (clamped
    // and scaled there, so a transfer only shifts and adds); every load of a
    // wavefront then reads the same one of a stage's two pages (kOnePage) or
    // picks per load.  Beyond that (LONG) the block ids are read through the
    // scalar data cache (constant address space: the table is read-only and
    // the index uniform), which is counted apart from the global->LDS
    // transfers but shares the LDS counter, so it is slightly slower.
    constexpr bool kOnePage = NW % (2 * BPP) == 0;
    const int pw = (wave / BPP) & 1;  // kOnePage: the page this wavefront loads
    typedef __attribute__((address_space(4))) const int32_t cint32_t;
    int bts = s;  // block-table row of the sequence
    if (SP) {
        bts = p.seq_row[s];
        bts = (bts >= 0 && bts < p.bt_rows) ? bts : 0;
    }
    const cint32_t* bt_row =
        (const cint32_t*)(p.block_tables + (int64_t)bts * p.max_blocks + first_page);
    if constexpr (!LONG) {
        for (int i = tid; i < 2 * nstage; i += blockDim.x) {
            const int id = p.block_tables[(int64_t)bts * p.max_blocks + first_page + min(i, npages - 1)];
            const int64_t b = (id >= 0 && id < p.num_blocks) ? id : 0;
            lds_bid[(i & 1) * kIdRow + (i >> 1)] = (uint32_t)((b * p.Hkv + g) * (Gm::PAGE / 256));
        }
        __syncthreads();
    }
    auto stage_ids = [&](int st) {
        if constexpr (LONG) {
            return int2{bt_row[2 * st], bt_row[min(2 * st + 1, npages - 1)]};
        } else if constexpr (kOnePage) {
            // wave-uniform: made scalar at once
            const int v = __builtin_amdgcn_readfirstlane((int)lds_bid[pw * kIdRow + st]);
            return int2{v, v};
        } else {
            return int2{__builtin_amdgcn_readfirstlane((int)lds_bid[st]),
                        __builtin_amdgcn_readfirstlane((int)lds_bid[kIdRow + st])};
        }
    };
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)lds;  // LDS byte address of the ring
    auto issue_stage = [&](int st, int2 ids) {
        uint8_t* base = lds + (st % NS) * Gm::STAGE;
        const uint32_t lbase = lds0 + (uint32_t)((st % NS) * Gm::STAGE);
        if constexpr (LONG) {
            const int64_t ba = (ids.x >= 0 && ids.x < p.num_blocks) ? ids.x : 0;
            const int64_t bb = (ids.y >= 0 && ids.y < p.num_blocks) ? ids.y : 0;
            const uint8_t* kA = kpool + ba * page_stride + head_off;
            const uint8_t* kB = kpool + bb * page_stride + head_off;
            const uint8_t* vA = vpool + ba * page_stride + head_off;
            const uint8_t* vB = vpool + bb * page_stride + head_off;
#pragma unroll
            for (int c = 0; c < Gm::LPT; ++c) {
                const int blk = c * NW + wave;
                const int buf = blk / BPP;             // 0 K a, 1 K b, 2 V a, 3 V b
                const uint8_t* src = buf == 0 ? kA : buf == 1 ? kB : buf == 2 ? vA : vB;
                load_to_lds16(src + src_off[c], base + blk * 1024);
            }
        } else {
            const uint64_t oa = (uint64_t)(uint32_t)ids.x << 8;
            const uint64_t ob = kOnePage ? oa : (uint64_t)(uint32_t)ids.y << 8;
#pragma unroll
            for (int c = 0; c < Gm::LPT; ++c) {
                const int blk = c * NW + wave;
                const int buf = blk / BPP;             // 0 K a, 1 K b, 2 V a, 3 V b
                const uint8_t* pool = (buf >> 1) ? vpool : kpool;
                load_to_lds16(pool + ((buf & 1) ? ob : oa), (uint32_t)src_off[c], lbase + blk * 1024);
            }
        }
    };

    // all-ones bf16 operand of the column-sum product, kept in registers
    u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    asm volatile("" : "+v"(ones));
    f32x4 acc[2][Gm::NT];
    f32x4 lsum[2];  // column sums of P, accumulated on the matrix cores
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        lsum[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < Gm::NT; ++t) acc[nt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m_run[2] = {-INFINITY, -INFINITY};
    // derived from m_run, updated only when it is raised: the threshold past
    // which a logit raises it, and the exponent offset -m_run (0 while no key
    // has been seen)
    float m_thr[2] = {-INFINITY, -INFINITY};
    float m_off[2] = {0.f, 0.f};

    // Per-lane LDS offsets inside the ring, fixed for the whole loop; they
    // include this wavefront's slot within a round (stage st sits in slot
    // st % NS = (round * SPLIT) % NS + half).
    const int hoff = SPLIT > 1 ? half * Gm::STAGE : 0;
    int koff[Gm::KCH];  // K operand: row col, chunk 4i + grp
#pragma unroll
    for (int i = 0; i < Gm::KCH; ++i)
        koff[i] = hoff + col * Gm::RB + swz_k<Gm::CPR>(col, 4 * i + grp) * 16;
    int voff[Gm::NT];   // bf16 V^T: row 4grp + col/4, columns 16t + 4(col%4) .. +3
    // (both also 64 KiB up, for slots past the 16-bit immediate offset of LDS
    // reads; kept opaque so that they stay in registers)
    int koff_hi[Gm::KCH], voff_hi[Gm::NT];
    {
        const int vrow = 4 * grp + (col >> 2);
        const int vsub = (col & 3) * 8;
#pragma unroll
        for (int t = 0; t < Gm::NT; ++t)
            voff[t] = hoff + vrow * Gm::RB + swz_v<Gm::CPR>(vrow, 2 * t + (vsub >> 4)) * 16 +
                      (vsub & 15);
    }
#pragma unroll
    for (int i = 0; i < Gm::KCH; ++i) {
        koff_hi[i] = koff[i] + 65536;
        asm volatile("" : "+v"(koff_hi[i]));
    }
#pragma unroll
    for (int t = 0; t < Gm::NT; ++t) {
        voff_hi[t] = voff[t] + 65536;
        asm volatile("" : "+v"(voff_hi[t]));
    }

    // One stage.  `slot_tag` is the compile-time ring slot of the round
    // (interior rounds, so every LDS address is a register plus an immediate)
    // or -1 (slot `dyn_slot`).  EDGE stages mask keys outside
    // [kv_start, position] and zero the V rows of keys outside
    // [kv_start, pos_max].  The running max is raised lazily: only when some
    // column's tile max exceeds it by more than 8 (log2 units); column sums of
    // P come from one extra MFMA against an all-ones operand.
    // `after_qk` runs once the logit products are issued (it reads the next
    // round's page offsets).
    auto compute = [&](auto edge_tag, auto slot_tag, int dyn_slot, int st, auto&& after_qk) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        constexpr int SLOT = decltype(slot_tag)::value;
        // slots from 64 KiB on use the offsets 64 KiB up and a smaller base
        constexpr bool HI = SLOT >= 0 && SLOT * Gm::STAGE >= 65536;
        const uint8_t* sb = lds + (SLOT >= 0 ? SLOT : dyn_slot) * Gm::STAGE - (HI ? 65536 : 0);
        const int* ko = HI ? koff_hi : koff;
        const int* vo = HI ? voff_hi : voff;
        const int pa = first_page + 2 * st;
        // ---- operands from LDS: K for the logits first.  The (bfloat16) V^T
        // operands are read only once the logit products are issued: right
        // after the barrier every wavefront of the workgroup reads its K, and
        // with the V^T reads queued behind them the second wavefront of a
        // SIMD would wait for the first one's V^T before its own K arrived.
        // Read later, their latency overlaps the softmax.
        u32x4 kop[2][Gm::KCH];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int i = 0; i < Gm::KCH; ++i)
                kop[x][i] = *reinterpret_cast<const u32x4*>(sb + x * Gm::PAGE + ko[i]);
        u32x4 vop[kBF ? Gm::NT : 1];
        mfma_priority(1);
        // ---- S^T tiles: keys of page x as rows, this wavefront's rows as columns.
        // The four tiles accumulate over the head dimension in four independent
        // chains, issued step by step across the chains (a scheduling barrier
        // after each step) so that a product never waits on the one just before
        // it: a dependent product issues only ~52 cycles after its predecessor,
        // four independent ones every 16.
        f32x4 sx[2][2];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) sx[nt][x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < Gm::KCH; ++i) {
            if constexpr (kBF) {
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        sx[nt][x] = mfma_bf16(kop[x][i], qop[nt][i], sx[nt][x]);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int x = 0; x < 2; ++x)
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
                            sx[nt][x] = mfma_f32(__uint_as_float(kop[x][i][t]),
                                                 __uint_as_float(qop[nt][i][t]), sx[nt][x]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kBF) {
#pragma unroll
            for (int t = 0; t < Gm::NT; ++t) {
                const uint2 lo = lds_read_tr16(sb + 2 * Gm::PAGE + vo[t]);
                const uint2 hi = lds_read_tr16(sb + 3 * Gm::PAGE + vo[t]);
                vop[t] = u32x4{lo.x, lo.y, hi.x, hi.y};
            }
        }
        after_qk();
        mfma_priority(0);
        bool kval[8];
        if constexpr (EDGE) {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int key = (pa + x) * kPage + grp * 4 + t;
                    kval[x * 4 + t] = key >= r.a && key <= pos_max;
                }
        }
        float sv[2][8];
        bool grow = false;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            float mt = -INFINITY;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    float v = sx[nt][x][t];
                    if constexpr (EDGE) {
                        const int key = (pa + x) * kPage + grp * 4 + t;
                        v = (key >= r.a && key <= pos[nt]) ? v : -INFINITY;
                    }
                    sv[nt][x * 4 + t] = v;
                    mt = fmaxf(mt, v);
                }
            grow |= mt * p.scale_log2 > m_thr[nt];
        }
        if (__any(grow)) {
            // exact column maxima, then rescale what was accumulated so far in
            // the columns that passed their threshold (the others keep their
            // state bit for bit, so a row's result never depends on its
            // neighbours in the tile)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                float mt = sv[nt][0];
#pragma unroll
                for (int t = 1; t < 8; ++t) mt = fmaxf(mt, sv[nt][t]);
                mt = col_max(mt) * p.scale_log2;
                const float m_new = mt > m_thr[nt] ? fmaxf(m_run[nt], mt) : m_run[nt];
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = fast_exp2(m_run[nt] - m_use);
                m_run[nt] = m_new;
                m_thr[nt] = m_new + 8.f;
                m_off[nt] = -m_use;
                lsum[nt] *= alpha;
#pragma unroll
                for (int t = 0; t < Gm::NT; ++t) acc[nt][t] *= alpha;
            }
        }
        u32x4 pb[2];
        float pv[2][8];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
                pv[nt][t] = fast_exp2(__builtin_fmaf(sv[nt][t], p.scale_log2, m_off[nt]));
            if constexpr (kBF)
                pb[nt] = u32x4{pack_bf16(pv[nt][0], pv[nt][1]), pack_bf16(pv[nt][2], pv[nt][3]),
                               pack_bf16(pv[nt][4], pv[nt][5]), pack_bf16(pv[nt][6], pv[nt][7])};
        }

        mfma_priority(1);
        // ---- O^T += V^T P^T, and the column sums of P
        if constexpr (kBF) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) lsum[nt] = mfma_bf16(ones, pb[nt], lsum[nt]);
            uint32_t keep[4];
            if constexpr (EDGE) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    keep[q] = (kval[2 * q] ? 0x0000ffffu : 0u) | (kval[2 * q + 1] ? 0xffff0000u : 0u);
            }
#pragma unroll
            for (int t = 0; t < Gm::NT; ++t) {
                u32x4 a = vop[t];
                if constexpr (EDGE) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) a[q] &= keep[q];
                }
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[nt][t] = mfma_bf16(a, pb[nt], acc[nt][t]);
            }
        } else {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int key = grp * 4 + u;
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        lsum[nt] = mfma_f32(1.f, pv[nt][x * 4 + u], lsum[nt]);
#pragma unroll
                    for (int t = 0; t < Gm::NT; ++t) {
                        const int dcol = t * 16 + col;
                        float v = *reinterpret_cast<const float*>(
                            sb + (HI ? 65536 : 0) + hoff + (2 + x) * Gm::PAGE + key * Gm::RB +
                            swz_v<Gm::CPR>(key, dcol >> 2) * 16 + (dcol & 3) * 4);
                        if constexpr (EDGE) v = kval[x * 4 + u] ? v : 0.f;
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
                            acc[nt][t] = mfma_f32(v, pv[nt][x * 4 + u], acc[nt][t]);
                    }
                }
        }
        mfma_priority(0);
    };

    // Round rr: stages rr * SPLIT .. rr * SPLIT + SPLIT - 1, one per wavefront
    // of a row block.  Before the barrier this thread's loads of those stages
    // are complete; after it every wavefront is done with round rr - 1, whose
    // slots take the stages NS - SPLIT ahead.
    // ids[j]: what the transfers of the next round's j-th stage need (page
    // offsets / 256, or block ids in the LONG variant)
    int2 ids[SPLIT];
    // Interior rounds (EDGE false) also lie far enough from the end that
    // every stage they wait for and issue exists: their wait is a constant and
    // their transfers are unconditional.
    auto round = [&](auto edge_tag, auto slot_tag, int rr) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        if constexpr (EDGE) {
            const int last_needed = min(rr * SPLIT + SPLIT - 1, nstage - 1);
            const int last_issued = min(rr * SPLIT + NS - SPLIT - 1, nstage - 1);
            wait_stages<Gm::LPT, NS - 2 * SPLIT>(last_issued - last_needed);
        } else {
            wait_vmcnt<(NS - 2 * SPLIT) * Gm::LPT>();
        }
        barrier_keep_loads_in_flight();
#pragma unroll
        for (int j = 0; j < SPLIT; ++j) {
            const int st = rr * SPLIT + NS - SPLIT + j;
            if (!EDGE || st < nstage) issue_stage(st, ids[j]);
        }
        if constexpr (!LONG) {
#pragma unroll
            for (int j = 0; j < SPLIT; ++j) {
                const int nx = rr * SPLIT + NS + j;
                if (EDGE) {
                    if (nx < nstage) ids[j] = stage_ids(nx);
                } else if constexpr (!(kOnePage && SPLIT == 2)) {
                    ids[j] = stage_ids(nx);  // inside the padded row; used only if it exists
                }
            }
        }
        // Interior rounds of the one-page layout read both stages of the next
        // round in one 8-byte read (an even index), issued after this round's
        // logit products and made scalar at the end of the round, so that its
        // LDS round trip never sits between the barrier and the K reads.
        constexpr bool kLateIds = !LONG && !EDGE && kOnePage && SPLIT == 2;
        uint2 next_ids;
        auto after_qk = [&]() {
            if constexpr (kLateIds)
                next_ids = *reinterpret_cast<const uint2*>(&lds_bid[pw * kIdRow + rr * SPLIT + NS]);
        };
        // (every stage of an interior round exists)
        const int st = rr * SPLIT + half;
        if (!EDGE || st < nstage) compute(edge_tag, slot_tag, (rr * SPLIT) % NS, st, after_qk);
        if constexpr (kLateIds) {
            const int a = __builtin_amdgcn_readfirstlane((int)next_ids.x);
            const int b = __builtin_amdgcn_readfirstlane((int)next_ids.y);
            ids[0] = int2{a, a};
            ids[1] = int2{b, b};
        }
        if constexpr (LONG) {
            // the next round's block ids, fetched after this round's LDS reads
            // so that their scalar-cache latency overlaps the barrier rather
            // than the reads (both are counted by lgkmcnt)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < SPLIT; ++j) {
                const int nx = rr * SPLIT + NS + j;
                if (nx < nstage) ids[j] = stage_ids(nx);
            }
        }
    };

    // the query operands have arrived before any staged load is issued, so
    // the vmcnt waits below count staged loads only
    wait_vmcnt<0>();
#pragma unroll
    for (int st = 0; st < NS - SPLIT; ++st)
        if (st < nstage) issue_stage(st, stage_ids(st));
#pragma unroll
    for (int j = 0; j < SPLIT; ++j)
        ids[j] = stage_ids(min(NS - SPLIT + j, nstage - 1));

    using Dyn = std::integral_constant<int, -1>;
    // Round 0 and every round past the interior take the masked path; interior
    // rounds (all keys in [kv_start, first position of the tile]) run unrolled
    // over the ring with compile-time slots.
    constexpr int U = NS / SPLIT;  // rounds per pass over the ring
    const int nround = (nstage + SPLIT - 1) / SPLIT;
    const int full = (pos_min - first_page * kPage - 2 * kPage + 1) < 0
                         ? 0 : (pos_min - first_page * kPage - 2 * kPage + 1) / (2 * kPage) + 1;
    // rounds [1, r_hi) are interior: every key of theirs lies in
    // [kv_start, first position of the tile], and every stage they issue,
    // up to rr * SPLIT + NS - 1, exists
    const int r_hi = min(min(nstage, full) / SPLIT, nstage >= NS ? (nstage - NS) / SPLIT + 1 : 0);
    round(std::true_type{}, Dyn{}, 0);
    int rr = 1;
    for (; rr + U - 1 < r_hi; rr += U) {
        unroll_rounds<0, U>([&](auto k) {
            constexpr int KK = decltype(k)::value;
            round(std::false_type{}, std::integral_constant<int, (SPLIT * (1 + KK)) % NS>{},
                  rr + KK);
        });
    }
    for (; rr < nround; ++rr) round(std::true_type{}, Dyn{}, rr);

    float l_tot[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) l_tot[nt] = lsum[nt][0];  // every row holds the column sum
    if constexpr (SPLIT > 1) {
        // the second wavefront of each row block hands (acc, sum, max) to the first
        __syncthreads();  // all reads of the ring are done; no loads in flight
        float* xch = reinterpret_cast<float*>(lds) + rblk * Gm::XF * kWave + lane;
        if (half != 0) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
                for (int t = 0; t < Gm::NT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xch[((nt * Gm::NT + t) * 4 + i) * kWave] = acc[nt][t][i];
                xch[(2 * Gm::NT * 4 + 2 * nt) * kWave] = l_tot[nt];
                xch[(2 * Gm::NT * 4 + 2 * nt + 1) * kWave] = m_run[nt];
            }
        }
        __syncthreads();
        if (half != 0) return;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const float l1 = xch[(2 * Gm::NT * 4 + 2 * nt) * kWave];
            const float m1 = xch[(2 * Gm::NT * 4 + 2 * nt + 1) * kWave];
            const float M = fmaxf(m_run[nt], m1);
            const float Mu = (M == -INFINITY) ? 0.f : M;
            const float a0 = fast_exp2(m_run[nt] - Mu);
            const float a1 = fast_exp2(m1 - Mu);
            l_tot[nt] = a0 * l_tot[nt] + a1 * l1;
            m_run[nt] = M;  // the combined state is relative to M
#pragma unroll
            for (int t = 0; t < Gm::NT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[nt][t][i] = a0 * acc[nt][t][i] + a1 * xch[((nt * Gm::NT + t) * 4 + i) * kWave];
        }
    }

#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        if (!rvalid[nt]) continue;
        if (SP) {
            // the softmax state of the row, unnormalised
            float* sr = p.state + orow_idx[nt] * kStateStride<D>;
#pragma unroll
            for (int t = 0; t < Gm::NT; ++t)
                *reinterpret_cast<f32x4*>(sr + t * 16 + grp * 4) = acc[nt][t];
            if (grp == 0) {
                sr[D] = m_run[nt];
                sr[D + 1] = l_tot[nt];
            }
            continue;
        }
        const float inv = l_tot[nt] > 0.f ? 1.f / l_tot[nt] : 0.f;
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

template <typename T, int D, bool LONG>
__global__ void __launch_bounds__(kPrefillThreads<T>) prefill_kernel(PrefillParams p) {
    __shared__ PrefillLds<T, D, LONG> lds;
    prefill_tile<T, D, LONG>(p, (int)blockIdx.x, lds);
}

}  // namespace pkv
